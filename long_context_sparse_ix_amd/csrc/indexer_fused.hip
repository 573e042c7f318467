// Full-layer indexer fused with a streaming per-row top-k (gfx950).
//
// What it computes ("IndexShare", LLM Architecture Gallery, section "Why The
// Indexer Becomes Expensive"; "GLM-5.2 and IndexShare for Long-Context Sparse
// Attention", section "Where the DSA indexer becomes expensive"): for each
// query row at position p, score every key s <= p with
//     score(p, s) = sum_h w[h] * max(0, q[h,:] . key[s,:])
// and keep the k best positions (equal scores: lower position), emitted in
// ascending position order and padded with -1.  The score matrix is never
// written anywhere: scores live in registers for one 64-key tile and only
// candidates that can still reach the top k are kept.
//
// Layout of the work
//   * one workgroup = 4 waves = 4 consecutive query rows (one row per wave),
//     two workgroups per CU (two waves per SIMD, so one wave's memory and LDS
//     waits overlap the other's MFMAs); row blocks are issued longest-first so
//     the causal triangle drains evenly;
//   * keys stream HBM -> LDS with direct loads (buffer_load_dwordx4 ... lds,
//     no VGPR staging) into a 4-slot ring of 64-key tiles (bf16, or e4m3fn
//     codes in the Q8 instance) shared by the 4 rows, rows XOR-swizzled so B-operand reads are bank-conflict free; tiles
//     are consumed in pairs, one LDS-only barrier per pair;
//   * each wave keeps its row's heads x d query slice in registers as the MFMA
//     A operand (M = heads) and reads 32-key halves of a tile as the B operand
//     (N = keys): v_mfma_f32_32x32x16_bf16, output lane l holds key l%32 and 16
//     heads.  Software pipeline by half tile: while the MFMAs of one half run,
//     the VALU does the epilogue of the other (ReLU, head weight, sum over the
//     lane's heads); one permlane32 swap + add completes the head sum and
//     leaves lane l with the score of key tile_start + l;
//   * streaming top-k per row: a strict "score > tau" filter appends survivors
//     to the row's candidate buffer in the workspace (L2-resident, ascending
//     position order).  At pair boundaries, when any row of the workgroup
//     nears capacity, the fuller rows shrink together: one histogram pass over
//     the score range picks the bin holding the k-th best and everything below
//     that bin is dropped; tau becomes the smallest kept score.  Because keys
//     arrive in ascending position, a later key tying tau always loses the
//     tie, so the strict filter is exact.  A crowded bin (ties) falls back to
//     an exact radix select;
//   * at the end an exact radix select (score desc, position asc) picks the k
//     winners and a stable pass writes their positions in ascending order.
//
// Queries declared as e4m3fn codes (one scale per row and head, IndexCache
// notes, section 1: an FP8 indexer) run the Q8 instance when the keys are
// e4m3fn too and d is 64 or 128: the tiles hold the cache's raw codes, read
// in place (no staging copy), and v_mfma_f32_32x32x64_f8f6f4 multiplies codes
// by codes; the query scale folds into the head weight and the key scale
// multiplies the finished head sum.  Other fp8-query forms widen the codes
// to bf16 in the prologue and run the bf16 instances.
//
// The same kernel with SELECT = false keeps only a running maximum per lane
// instead of the candidate buffer: the row's best position (equal scores:
// lower position) and its score, i.e. the top-1 under the same rule.  It
// streams the same scores through the same tile ring and MFMA pipeline, so
// its time is the score stream's alone and the difference to the full kernel
// is what the streaming top-k costs.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kTileKeys = 64;
constexpr int kRowsPerWG = 4;
constexpr int kThreads = kRowsPerWG * kWave;
constexpr int kRing = 4;        // LDS tile buffers: a pair of tiles being read, the next pair landing
constexpr int kUnroll = 8;      // (score, position) entries per lane in flight in buffer passes
constexpr int kUnrollS = 16;    // scores per lane in flight in score-only passes

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// buffer resource word 3 for raw (unformatted, unswizzled) 32-bit data on CDNA
constexpr int kRsrcWord3 = 0x00020000;

// Wait until at most N of this wave's vector-memory operations are
// outstanding (direct-to-LDS loads are invisible to the compiler's waitcnt
// tracking, so the tile ring waits explicitly).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only.  __syncthreads() also drains every
// outstanding global access of the wave (vmcnt(0)), which would wait for the
// tile prefetched two steps ahead; the ring's own vmcnt waits cover global ->
// LDS data, and candidate-buffer stores are private to their wave.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Thresh {
  uint32_t v;   // order key of the k-th best entry
  int need;     // how many entries with key == v belong to the top k
};

__device__ __forceinline__ float wave_min_f(float v) { return wave_min(v); }
__device__ __forceinline__ float wave_max_f(float v) { return wave_max(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_min(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_max(v); }

// Candidate buffer of one row: `cap` scores, then the `cap` positions (two
// arrays, so passes that need only the scores read contiguous words).  Passes
// load from indices clamped into the buffer and mask the values afterwards:
// unconditional loads let one wait cover a whole batch of them.
struct Cand {
  float* s;
  int32_t* p;
  int cap;
  __device__ __forceinline__ int at(int i) const { return min(i, cap - 1); }
};

// Bin holding the kk-th largest entry of a 256-bin LDS histogram (lane l owns
// bins 4l..4l+3).  Returns the bin; `above` = entries in higher bins, `in_bin`
// = entries in the bin.
__device__ __forceinline__ int pick_bin(const uint32_t* hist, int kk, int& above, int& in_bin) {
  const int l = lane_id();
  const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
  const uint32_t tot = h.x + h.y + h.z + h.w;
  const int a3 = (int)(wave_suffix_sum(tot) - tot);   // entries in higher lanes' bins
  const int a2 = a3 + (int)h.w, a1 = a2 + (int)h.z, a0 = a1 + (int)h.y;
  int bin = -1, ab = 0, cb = 0;
  if (a3 < kk && kk <= a2) { bin = 4 * l + 3; ab = a3; cb = (int)h.w; }
  else if (a2 < kk && kk <= a1) { bin = 4 * l + 2; ab = a2; cb = (int)h.z; }
  else if (a1 < kk && kk <= a0) { bin = 4 * l + 1; ab = a1; cb = (int)h.y; }
  else if (a0 < kk && kk <= a0 + (int)h.x) { bin = 4 * l; ab = a0; cb = (int)h.x; }
  const uint64_t m = __ballot(bin >= 0);
  const int src = __ffsll((unsigned long long)m) - 1;
  above = __shfl(ab, src);
  in_bin = __shfl(cb, src);
  return __shfl(bin, src);
}

__device__ __forceinline__ void clear_hist(uint32_t* hist) {
  *reinterpret_cast<u32x4*>(hist + 4 * lane_id()) = u32x4{0u, 0u, 0u, 0u};
  wave_lds_sync();
}

__device__ __forceinline__ int range_bits8(uint32_t range) {   // bit length rounded up to 8
  const int nbits = range == 0u ? 0 : 32 - __clz((int)range);
  return (nbits + 7) & ~7;
}

// Exact k-th best among the cnt >= k >= 1 entries (score desc): radix select
// on order-key offsets from the minimum, 8 bits per pass from the top of the
// key range.
__device__ Thresh select_kth(Cand c, int cnt, int k, uint32_t* hist) {
  const int l = lane_id();
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int base = 0; base < cnt; base += kWave * kUnrollS) {
    float v[kUnrollS];
#pragma unroll
    for (int u = 0; u < kUnrollS; ++u) v[u] = c.s[c.at(base + u * kWave + l)];
#pragma unroll
    for (int u = 0; u < kUnrollS; ++u)
      if (base + u * kWave + l < cnt) {
        const uint32_t key = order_key(v[u]);
        lo = min(lo, key);
        hi = max(hi, key);
      }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  for (int shift = range_bits8(hi - lo) - 8; shift >= 0; shift -= 8) {
    clear_hist(hist);
    for (int base = 0; base < cnt; base += kWave * kUnrollS) {
      float v[kUnrollS];
#pragma unroll
      for (int u = 0; u < kUnrollS; ++u) v[u] = c.s[c.at(base + u * kWave + l)];
#pragma unroll
      for (int u = 0; u < kUnrollS; ++u) {
        const uint32_t rel = order_key(v[u]) - lo;
        if (base + u * kWave + l < cnt && (rel & pmask) == prefix)
          atomicAdd(&hist[(rel >> shift) & 255u], 1u);
      }
    }
    wave_lds_sync();
    int above, in_bin;
    const int b = pick_bin(hist, kk, above, in_bin);
    kk -= above;
    prefix |= (uint32_t)b << shift;
    pmask |= 0xFFu << shift;
  }
  return Thresh{lo + prefix, kk};
}

// Stable pass over the buffer keeping key > t.v and the first t.need entries
// with key == t.v (the lowest positions: the buffer is in position order).
// EMIT: write the kept positions to dst; otherwise compact in place and
// return the new count.  In place is safe: every chunk is read before any of
// its slots can be overwritten, and writes never pass the chunk being read.
template <bool EMIT>
__device__ int keep_pass(Cand c, int cnt, Thresh t, int32_t* dst, int limit = 0) {
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  for (int base = 0; base < cnt; base += kWave * kUnroll) {
    float v[kUnroll];
    int32_t pos[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = c.at(base + u * kWave + l);
      v[u] = c.s[i];
      pos[u] = c.p[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool in = base + u * kWave + l < cnt;
      const uint32_t key = order_key(v[u]);
      const bool eq = in && key == t.v;
      const uint64_t em = __ballot(eq);
      const bool keep = (in && key > t.v) || (eq && eq_seen + wave_prefix(em) < t.need);
      const uint64_t km = __ballot(keep);
      if (keep) {
        const int o = out + wave_prefix(km);
        if constexpr (EMIT) {
          if (o < limit) dst[o] = pos[u];        // exactly limit entries are kept
        } else {
          c.s[o] = v[u];
          c.p[o] = pos[u];
        }
      }
      out += __popcll(km);
      eq_seen += __popcll(em);
    }
  }
  return out;
}

// Buffer shrink during the stream, in the score-value domain.  One histogram
// over [lo, hi] (lo: a lower bound of every entry, hi: the largest entry)
// gives the bin b holding the k-th best; every entry in bins >= b is kept.
// The bin map is monotone in the score, so the kept set is {s >= s*} with at
// least k members: the k-th best is >= s*, nothing below s* can win, and a
// later key equal to s* loses the position tie, so tau = s* keeps the strict
// filter exact.  A crowded bin (ties, or a range too wide to split) falls back
// to the exact select.
__device__ __forceinline__ void shrink(Cand c, int& cnt, float& tau, float hi_lane, float lo_lane, int k,
                                       int keep_max, uint32_t* hist) {
  const int l = lane_id();
  wait_vmcnt<0>();                               // this wave's appends are visible
  const float hi = wave_max_f(hi_lane);
  // every entry is above tau once a shrink has set it; before that the
  // buffer holds exactly the appends, whose minimum each lane tracked
  const float lo = tau == -INFINITY ? wave_min_f(lo_lane) : tau;
  const float inv = 256.0f / (hi - lo);
  if (hi > lo && inv > 0.0f && inv < INFINITY) {
    clear_hist(hist);
    for (int base = 0; base < cnt; base += kWave * kUnrollS) {
      float v[kUnrollS];
#pragma unroll
      for (int u = 0; u < kUnrollS; ++u) v[u] = c.s[c.at(base + u * kWave + l)];
#pragma unroll
      for (int u = 0; u < kUnrollS; ++u)
        if (base + u * kWave + l < cnt) atomicAdd(&hist[min(255, max(0, (int)((v[u] - lo) * inv)))], 1u);
    }
    wave_lds_sync();
    int above, in_bin;
    const int b = pick_bin(hist, k, above, in_bin);
    if (above + in_bin <= keep_max) {
      int out = 0;
      float smin = INFINITY;
      for (int base = 0; base < cnt; base += kWave * kUnroll) {
        float v[kUnroll];
        int32_t pos[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int i = c.at(base + u * kWave + l);
          v[u] = c.s[i];
          pos[u] = c.p[i];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const bool keep = base + u * kWave + l < cnt && min(255, max(0, (int)((v[u] - lo) * inv))) >= b;
          const uint64_t km = __ballot(keep);
          if (keep) {
            const int o = out + wave_prefix(km);
            c.s[o] = v[u];
            c.p[o] = pos[u];
            smin = fminf(smin, v[u]);
          }
          out += __popcll(km);
        }
      }
      cnt = out;
      tau = wave_min_f(smin);
      return;
    }
  }
  const Thresh th = select_kth(c, cnt, k, hist);
  cnt = keep_pass<false>(c, cnt, th, nullptr);
  tau = key_value(th.v);
}

// Key tile in LDS: 64 rows of d bf16 (CPR = d/8 16-byte chunks per row),
// unpadded, with chunk c of row r stored in slot c ^ f(r), f(r) = (r / RPB) %
// CPR where RPB = 16 / CPR rows share one 256-byte bank cycle.  The 16 rows a
// B-operand read touches then land in 16 distinct bank groups.
template <int KS>
struct TileGeom {
  static constexpr int d = KS * 16;
  static constexpr int CPR = d / 8;
  static constexpr int RPB = 16 / CPR;
  static constexpr int row_bytes = d * 2;
  static constexpr int tile_bytes = kTileKeys * row_bytes;
  static constexpr int inst_per_wave = CPR >= 4 ? CPR / 4 : 1;      // 16-byte direct loads per wave
  static constexpr int lanes_per_inst = CPR >= 4 ? 64 : 16 * CPR;
  static_assert(CPR == 2 || CPR == 4 || CPR == 8 || CPR == 16, "d must be 16, 32, 64 or 128");
  __device__ static __forceinline__ int swz(int r, int c) { return c ^ ((r / RPB) & (CPR - 1)); }
};

template <int KS>
__device__ __forceinline__ void read_bfrags(const unsigned char* kb, int nt, int m, int hf, bf16x8 (&bfr)[KS]) {
  using G = TileGeom<KS>;
  const int r = nt * 32 + m;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bfr[ks] = *reinterpret_cast<const bf16x8*>(kb + r * G::row_bytes + G::swz(r, hf * (G::CPR / 2) + ks) * 16);
}

// Two 16-byte B chunks as one fp8 MFMA operand (32 codes).
__device__ __forceinline__ i32x8 join_b(const bf16x8& lo, const bf16x8& hi) {
  const u32x4 x = __builtin_bit_cast(u32x4, lo), y = __builtin_bit_cast(u32x4, hi);
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// One half-tile block: the MFMAs of one 32-key half into acc_mma and/or the
// epilogue of the other accumulator half (acc_epi), in one basic block so the
// scheduler can put the VALU work between MFMAs.  Returns the partial (this
// lane's heads) score of the epilogue half.  AF = bf16x8: NA = NB k-steps of
// v_mfma_f32_32x32x16_bf16.  AF = i32x8 (e4m3fn codes): NA k-steps of
// v_mfma_f32_32x32x64_f8f6f4, each taking B chunks 2kk and 2kk+1 (the A
// fragment holds the same 32 dims of the query as those two key chunks).
template <int HT, int NA, int NB, bool MMA, bool EPI, typename AF>
__device__ __forceinline__ float half_block(const AF (&qf)[HT][NA], const float (&wr)[HT][16],
                                            const bf16x8 (&bfr)[NB], f32x16 (&acc_mma)[HT],
                                            const f32x16 (&acc_epi)[HT]) {
  constexpr bool kF8 = std::is_same<AF, i32x8>::value;
  static_assert(kF8 ? NB == 2 * NA : NB == NA, "B chunks per A fragment");
  if constexpr (MMA) {
    // a wave issuing MFMAs outranks the other wave of its SIMD while that one
    // filters or shrinks, so the matrix pipe stays fed (0.7% at L=128K)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < NA; ++ks) {
      if constexpr (kF8) {
        const i32x8 bb = join_b(bfr[2 * ks], bfr[2 * ks + 1]);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)   // format 0 (e4m3) for A and B, no block scales
          acc_mma[ht] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              qf[ht][ks], bb, ks == 0 ? f32x16{} : acc_mma[ht], 0, 0, 0, 0, 0, 0);
      } else {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc_mma[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][ks], bfr[ks],
                                                                ks == 0 ? f32x16{} : acc_mma[ht], 0, 0, 0);
      }
    }
  }
  float part = 0.0f;
  if constexpr (EPI) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};     // 4 independent chains
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r & 3] = fmaf(wr[ht][r], relu(acc_epi[ht][r]), s[r & 3]);
    part = (s[0] + s[1]) + (s[2] + s[3]);
  }
  if constexpr (MMA && EPI) {
    // an fp8 MFMA is twice a bf16 one's cycles for four times its k-steps
    constexpr int kValu = kF8 ? 32 / NA : 4;
#pragma unroll
    for (int i = 0; i < HT * NA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);                      // VALU
    }
  }
  if constexpr (MMA) __builtin_amdgcn_s_setprio(0);
  return part;
}

// Q8: e4m3fn queries times e4m3fn keys on the fp8 MFMA.  A key tile then
// holds the raw codes (d bytes a row, the geometry of a d/2-wide bf16 tile),
// loaded straight from the key cache; the per-key scale multiplies the head
// sum and the per-(row, head) query scale is folded into the head weight.
template <int HT, int KS, bool SCALE, bool SELECT, bool Q8>
__global__ __launch_bounds__(kThreads, 2) void fused_indexer_topk_kernel(FusedArgs a) {
  static_assert(!Q8 || ((KS == 4 || KS == 8) && SCALE), "fp8 MFMA form: d in {64, 128}, scaled keys");
  using G = TileGeom<Q8 ? KS / 2 : KS>;
  constexpr int d = KS * 16;                  // query / key dims
  constexpr int NA = Q8 ? KS / 4 : KS;        // A fragments (k-steps) per head tile
  constexpr int NB = G::CPR / 2;              // 16-byte B chunks per lane per 32-key half
  using AF = typename std::conditional<Q8, i32x8, bf16x8>::type;
  constexpr int kLoads = G::inst_per_wave + (SCALE ? 1 : 0);   // direct loads per wave per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* key_lds0 = smem;                                                   // [3][tile]
  float* scale_lds = reinterpret_cast<float*>(smem + kRing * G::tile_bytes);       // [3][64]
  uint32_t* hist = reinterpret_cast<uint32_t*>(scale_lds + kRing * kTileKeys);     // [4][256]
  int* fill_lds = reinterpret_cast<int*>(hist + kRowsPerWG * 256);                 // [2][4] buffer fills

  const int tid = threadIdx.x, wave = uniform(tid >> 6), l = tid & 63;
  const int m = l & 31, hf = l >> 5;
  const int b = blockIdx.y;
  const int row0 = (gridDim.x - 1 - blockIdx.x) * kRowsPerWG;
  const int t = row0 + wave;
  const bool row_ok = t < a.n_q;
  const int qs = uniform((int)seq_start(a.seq_q_start, b, a.q_start));   // positions fit in int32
  const int p = qs + (row_ok ? t : 0);
  const int last_row = min(row0 + kRowsPerWG - 1, a.n_q - 1);
  const int n_keys = qs + last_row + 1;
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  const int C = a.C;
  float* const cand_base = reinterpret_cast<float*>(a.cand) + ((int64_t)b * a.n_q + (row_ok ? t : 0)) * 2 * C;
  const Cand cand{cand_base, reinterpret_cast<int32_t*>(cand_base + C), C};
  uint32_t* my_hist = hist + wave * 256;

  // Query slice (A operand): lane (m, hf) holds head ht*32+m, elements
  // [hf*d/2 + 8*ks, +8) of d for bf16 k-step ks, or codes [hf*d/2 + 32*ks,
  // +32) for fp8 k-step ks.  The key B operand uses the same element split,
  // so each dot product runs over all d elements.  e4m3fn queries outside
  // the fp8 MFMA form are widened exactly to bf16; their per-head scale is
  // folded into the head weight.
  AF qf[HT][NA];
  float wr[HT][16];
  {
    const int64_t qr = ((int64_t)b * a.n_q + (row_ok ? t : 0)) * a.H;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + m;
      const bool ok = row_ok && h < a.H;
      if constexpr (Q8) {
        const uint8_t* src = a.q8 + (qr + h) * d + hf * (d / 2);
#pragma unroll
        for (int ks = 0; ks < NA; ++ks) qf[ht][ks] = ok ? *reinterpret_cast<const i32x8*>(src + 32 * ks) : i32x8{};
      } else if (a.q8) {
        const uint8_t* src = a.q8 + (qr + h) * d + hf * (d / 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (ok) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(src + 8 * ks);
            const u32x2 lo = e4m3x4_to_bf16x4(c.x), hi = e4m3x4_to_bf16x4(c.y);
            v = u32x4{lo.x, lo.y, hi.x, hi.y};
          }
          qf[ht][ks] = __builtin_bit_cast(bf16x8, v);
        }
      } else {
        const uint16_t* qrow = a.q + qr * d;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[ht][ks] = ok ? *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * d + hf * (d / 2) + 8 * ks)
                          : bf16x8{};
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hh = ht * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);   // MFMA output row of acc[r]
        wr[ht][r] = (row_ok && hh < a.H)
                        ? a.w[qr + hh] * (a.q_scale ? a.q_scale[qr + hh] : 1.0f)
                        : 0.0f;
      }
    }
  }

  const float* scale_b = SCALE ? a.scale + (int64_t)b * a.scale_bstride : nullptr;

  // Direct HBM -> LDS loads of tile `it` into ring slot `slot`: load j of this
  // wave fills LDS slots [J*n, J*n+n) (J = wave + 4j, n lanes) in lane order, so
  // lane l fetches the global chunk that belongs in slot J*n + l (tile row r,
  // chunk swz(r, slot % CPR); swz is an involution).  With several loads per
  // wave (tiles of 8 KB and more) load j covers the 4 KB after load j-1 and
  // the swizzle repeats, so one per-lane byte offset serves all of them.  The
  // rows of the last, partial tile past the last key are masked; those past
  // the key array's kv_rows lie outside the load's resource and read zeros.
  static_assert(G::inst_per_wave == 1 || G::lanes_per_inst * 4 * 16 == 4096, "4 KB per load round");
  const int key_off = [&] {
    const int S = wave * G::lanes_per_inst + l;
    const int r = S / G::CPR;
    return r * G::row_bytes + G::swz(r, S % G::CPR) * 16;
  }();
  // The loads are buffer loads through a resource based at the tile (the
  // flat form, global_load_lds, makes the compiler treat every outstanding
  // one as an LDS access too, so each LDS read's wait became lgkmcnt(0)).
  const unsigned char* key_bytes;
  if constexpr (Q8) key_bytes = a.keys8 + (int64_t)b * a.key_bstride;
  else key_bytes = reinterpret_cast<const unsigned char*>(a.keys + (int64_t)b * a.key_bstride);
  auto issue_tile = [&](int it, int slot) {
    const int s0 = it * kTileKeys;
    // the staged copy is padded by a tile, so its tiles load whole; the key
    // cache read in place ends at kv_rows (>= 1 rows past s0: tiles start
    // below the last key)
    int tile_rows = kTileKeys;
    if constexpr (Q8) {
      const int64_t rows_left = a.kv_rows - s0;
      if (rows_left < kTileKeys) tile_rows = (int)rows_left;
    }
    unsigned char* tb = key_lds0 + slot * G::tile_bytes;
    const unsigned char* tile = key_bytes + (int64_t)s0 * G::row_bytes;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)tile, (short)0, tile_rows * G::row_bytes, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < G::inst_per_wave; ++j) {
      const int J = wave + 4 * j;
      if (G::lanes_per_inst == 64 || l < G::lanes_per_inst)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(tb + J * G::lanes_per_inst * 16), 16,
                                                 key_off + 4096 * j, 0, 0, 0);
    }
    if constexpr (SCALE) {
      const __amdgpu_buffer_rsrc_t sr =
          __builtin_amdgcn_make_buffer_rsrc((void*)(scale_b + s0), (short)0, tile_rows * 4, kRsrcWord3);
      if (l < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(scale_lds + slot * kTileKeys + 16 * wave), 4,
                                                 (16 * wave + l) * 4, 0, 0, 0);
    }
  };

  float tau = -INFINITY, vmax = -INFINITY, vmin = INFINITY;
  int cnt = 0;
  float best_s = -INFINITY;                     // SELECT == false: this lane's running maximum
  int best_p = -1;
  // Shrinks happen at pair boundaries, together: a pair appends at most 128
  // entries per row, so a row needs one when it holds more than C - 128; then
  // every row of the workgroup past `join` shrinks in the same step.  The rows
  // fill at similar rates, and the barrier makes the others wait for a
  // shrinking row anyway, so shrinking together turns the workgroup's stalls
  // from the sum of its rows' shrinks into about their maximum.  A shrink
  // keeps at most keep_max entries, so the next one is >= 128 appends away.
  const int keep_max = C - 4 * kWave;
  const int join = a.k + (C - a.k) / 2;
  float sc_prev = 1.0f;
  float part0 = 0.0f;                           // key-half-0 partial score of the tile being finished

  issue_tile(0, 0);
  if (n_tiles > 1) issue_tile(1, 1);
  wait_vmcnt<0>();
  __syncthreads();

  // Tiles are consumed in pairs with one barrier per pair: tile t sits in ring
  // slot t % 4; while the pair (it, it+1) is read, the pair (it+2, it+3) lands.
  f32x16 acc0[HT], acc1[HT];
  auto step = [&](int it, bool issue_pair) {
    const bool mma = row_ok && it < n_tiles && it * kTileKeys <= p;
    const bool epi = row_ok && it >= 1 && (it - 1) * kTileKeys <= p;
    const int slot = it & (kRing - 1);
    const unsigned char* kb = key_lds0 + slot * G::tile_bytes;
    // B operand of half 0 first (a stale, unused read when !mma), so its LDS
    // latency hides behind the tile issue
    bf16x8 bfr[NB];
    read_bfrags<NB>(kb, 0, m, hf, bfr);
    const float sc_cur = SCALE ? scale_lds[slot * kTileKeys + l] : 1.0f;
    if (issue_pair) {
      if (it + 2 < n_tiles) issue_tile(it + 2, (it + 2) & (kRing - 1));
      if (it + 3 < n_tiles) issue_tile(it + 3, (it + 3) & (kRing - 1));
    }

    // block X: MFMAs of half 0 of tile it || epilogue of half 1 of tile it-1
    float part1 = 0.0f;
    if (mma && epi) part1 = half_block<HT, NA, NB, true, true>(qf, wr, bfr, acc0, acc1);
    else if (mma) half_block<HT, NA, NB, true, false>(qf, wr, bfr, acc0, acc1);
    else if (epi) part1 = half_block<HT, NA, NB, false, true>(qf, wr, bfr, acc0, acc1);
    read_bfrags<NB>(kb, 1, m, hf, bfr);          // half 1, in flight during the finish

    if (epi) {
      // finish tile it-1: lanes 0-31 take key half 0, lanes 32-63 half 1
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1),
                                                       false, false);
      float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (SCALE) score *= sc_prev;
      const int s = (it - 1) * kTileKeys + l;
      if (s > p) score = -INFINITY;
      if constexpr (SELECT) {
        const bool pass = score > tau;           // room for 64: see the shrink below
        const uint64_t pm = __ballot(pass);
        if (pm) {
          if (pass) {
            const int o = cnt + wave_prefix(pm);
            cand.s[o] = score;
            cand.p[o] = s;
            vmax = fmaxf(vmax, score);            // per lane; reduced when a shrink needs it
            vmin = fminf(vmin, score);
          }
          cnt += __popcll(pm);
        }
      } else if (score > best_s) {               // keys arrive in ascending position:
        best_s = score;                          // strict > keeps the lowest of equal scores
        best_p = s;
      }
    }
    // block Y: MFMAs of half 1 of tile it || epilogue of its half 0
    if (mma) part0 = half_block<HT, NA, NB, true, true>(qf, wr, bfr, acc1, acc0);
    sc_prev = sc_cur;
  };
  for (int it = 0, parity = 0; it <= n_tiles; it += 2, parity ^= 1) {
    step(it, true);
    if (it + 1 <= n_tiles) step(it + 1, false);
    if constexpr (SELECT) {
      // post this row's fill; the slots alternate by pair so that a wave
      // already in the next pair cannot overwrite a fill still being read
      if (l == 0) fill_lds[parity * kRowsPerWG + wave] = cnt;
    }
    wait_vmcnt<0>();                             // the next pair landed
    lds_barrier();
    if constexpr (SELECT) {
      const int4 f = *reinterpret_cast<const int4*>(fill_lds + parity * kRowsPerWG);
      const int fullest = max(max(f.x, f.y), max(f.z, f.w));
      if (fullest > C - 2 * kWave && cnt > join) shrink(cand, cnt, tau, vmax, vmin, a.k, keep_max, my_hist);
    }
  }

  if constexpr (!SELECT) {
    // the row's best: the largest lane maximum, the lowest position among
    // lanes holding it (every row has its own key, so some lane holds one)
    const float bs = wave_max_f(best_s);
    const int bp = (int)wave_min_u32(best_s == bs ? (uint32_t)best_p : 0xFFFFFFFFu);
    if (row_ok && l == 0) {
      const int64_t r = (int64_t)b * a.n_q + t;
      a.idx[r] = bp;
      if (a.best) a.best[r] = bs;
    }
    return;
  }
  if (row_ok) {
    int32_t* dst = a.idx + ((int64_t)b * a.n_q + t) * a.k;
    wait_vmcnt<0>();
    int written;
    if (cnt > a.k) {
      const Thresh th = select_kth(cand, cnt, a.k, my_hist);
      keep_pass<true>(cand, cnt, th, dst, a.k);
      written = a.k;
    } else {
      for (int i = l; i < cnt; i += kWave) dst[i] = cand.p[i];
      written = cnt;
    }
    for (int i = written + l; i < a.k; i += kWave) dst[i] = -1;
  }
}

__global__ void stage_keys_kernel(const void* __restrict__ src, int fp8, int64_t src_bstride,
                                  const float* __restrict__ scale, int64_t scale_bstride,
                                  uint16_t* __restrict__ dst, float* __restrict__ dst_scale, int64_t rows,
                                  int64_t rows_padded, int d, int64_t total_chunks) {
  // one 16-element chunk per thread per step; d % 16 == 0 keeps chunks inside rows
  const int64_t chunks_per_row = d / 16;
  const int64_t per_seq = rows_padded * chunks_per_row;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = c / per_seq, rc = c % per_seq;
    const int64_t r = rc / chunks_per_row, off = (rc % chunks_per_row) * 16;
    u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
    if (r < rows) {
      if (fp8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(src) + b * src_bstride + r * d + off);
        u32x2 t;
        t = e4m3x4_to_bf16x4(v.x); o0.x = t.x; o0.y = t.y;
        t = e4m3x4_to_bf16x4(v.y); o0.z = t.x; o0.w = t.y;
        t = e4m3x4_to_bf16x4(v.z); o1.x = t.x; o1.y = t.y;
        t = e4m3x4_to_bf16x4(v.w); o1.z = t.x; o1.w = t.y;
      } else {
        const u32x4* v = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + b * src_bstride + r * d + off);
        o0 = v[0];
        o1 = v[1];
      }
    }
    u32x4* dd = reinterpret_cast<u32x4*>(dst + b * rows_padded * d + r * d + off);
    dd[0] = o0;
    dd[1] = o1;
    if (dst_scale && off == 0) dst_scale[b * rows_padded + r] = r < rows ? scale[b * scale_bstride + r] : 0.0f;
  }
}

template <int HT, int KS, bool SCALE, bool SELECT, bool Q8 = false>
hipError_t launch_fused_s(const FusedArgs& a, int B, hipStream_t s) {
  const size_t lds = fused_lds_bytes((Q8 ? KS / 2 : KS) * 16);   // an fp8 row is half a bf16 row
  const void* fn = reinterpret_cast<const void*>(&fused_indexer_topk_kernel<HT, KS, SCALE, SELECT, Q8>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((a.n_q + kRowsPerWG - 1) / kRowsPerWG, B);
  hipLaunchKernelGGL((fused_indexer_topk_kernel<HT, KS, SCALE, SELECT, Q8>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int HT, int KS, bool SELECT>
hipError_t launch_fused_t(const FusedArgs& a, int B, hipStream_t s) {
  return a.scale ? launch_fused_s<HT, KS, true, SELECT>(a, B, s) : launch_fused_s<HT, KS, false, SELECT>(a, B, s);
}

}  // namespace

int fused_candidates(int k) {
  const int extra = k > 4 * kWave ? k : 4 * kWave;
  return ((k + extra + kWave - 1) / kWave) * kWave;
}

size_t fused_lds_bytes(int d) {
  return (size_t)kRing * kTileKeys * 2 * d + kRing * kTileKeys * sizeof(float) +
         kRowsPerWG * 256 * sizeof(uint32_t) + 2 * kRowsPerWG * sizeof(int);
}

bool fused_dim_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

template <bool SELECT>
hipError_t launch_fused_sel(const FusedArgs& a, int B, int d, hipStream_t s) {
  const int HT = a.H > 32 ? 2 : 1;
  const int KS = d / 16;
  if (a.keys8) {
    if (!a.q8 || !a.scale || a.keys || a.kv_rows < 1) return hipErrorInvalidValue;
#define IX_FUSED_Q8(ht, ks) \
  if (HT == ht && KS == ks) return launch_fused_s<ht, ks, true, SELECT, true>(a, B, s);
    IX_FUSED_Q8(1, 4) IX_FUSED_Q8(1, 8) IX_FUSED_Q8(2, 4) IX_FUSED_Q8(2, 8)
#undef IX_FUSED_Q8
    return hipErrorInvalidValue;
  }
#define IX_FUSED_CASE(ht, ks) \
  if (HT == ht && KS == ks) return launch_fused_t<ht, ks, SELECT>(a, B, s);
  IX_FUSED_CASE(1, 1) IX_FUSED_CASE(1, 2) IX_FUSED_CASE(1, 4) IX_FUSED_CASE(1, 8)
  IX_FUSED_CASE(2, 1) IX_FUSED_CASE(2, 2) IX_FUSED_CASE(2, 4) IX_FUSED_CASE(2, 8)
#undef IX_FUSED_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_fused_indexer(const FusedArgs& a, int B, int d, hipStream_t s) {
  return launch_fused_sel<true>(a, B, d, s);
}

hipError_t launch_fused_argmax(const FusedArgs& a, int B, int d, hipStream_t s) {
  return launch_fused_sel<false>(a, B, d, s);
}

hipError_t launch_stage_keys(const void* src, bool fp8, int64_t src_bstride, const float* scale,
                             int64_t scale_bstride, uint16_t* dst, float* dst_scale, int B, int64_t rows,
                             int64_t rows_padded, int d, hipStream_t s) {
  const int64_t total = (int64_t)B * rows_padded * (d / 16);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(stage_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, fp8 ? 1 : 0, src_bstride,
                     scale, scale_bstride, dst, dst_scale, rows, rows_padded, d, total);
  return hipGetLastError();
}

}  // namespace ix
