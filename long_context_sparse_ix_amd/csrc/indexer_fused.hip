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
//   * one workgroup = 4 waves = 4 consecutive query rows (one row per wave);
//     row blocks are issued longest-first so the causal triangle drains evenly;
//   * keys stream through LDS in 64-key bf16 tiles (double-buffered, one
//     barrier per tile) shared by the 4 rows; the next tile's global loads are
//     in flight while the current one is consumed;
//   * each wave keeps its row's heads x d query slice in VGPRs as the MFMA A
//     operand (M = heads) and reads key tiles as the B operand (N = keys):
//     v_mfma_f32_32x32x16_bf16, output lane l holds key l%32 and 16 heads.
//     All B operands of a tile are read from LDS before its first MFMA;
//   * software pipeline: while tile i's MFMAs run, the VALU finishes tile
//     i-1 (ReLU, head weight, sum over the lane's heads; one permlane32 swap +
//     add completes the head sum and leaves lane l with the score of key
//     tile_start + l), so the epilogue hides under the matrix pipe;
//   * streaming top-k per row: a strict "score > tau" filter appends survivors
//     to a wave-private LDS candidate buffer kept in ascending position order.
//     When any row of the workgroup nears capacity, every row compacts at the
//     same barrier (one stall per workgroup, not one per row): one histogram
//     pass over the buffer's key range finds a bin edge T with at least k
//     entries >= T, entries below T are dropped and tau becomes T.  Because
//     keys arrive in ascending position, a later key tying tau always loses the
//     tie, so the strict filter is exact.  If a bin is too crowded (many equal
//     scores) the exact select below is used instead;
//   * at the end an exact radix select (score desc, position asc) picks the k
//     winners and a stable pass writes their positions in ascending order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kTileKeys = 64;
constexpr int kRowsPerWG = 4;
constexpr int kThreads = kRowsPerWG * kWave;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N of this wave's vector-memory loads are outstanding
// (direct-to-LDS loads are invisible to the compiler's own waitcnt tracking).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct Thresh {
  uint32_t v;   // order key of the k-th best entry
  int need;     // how many entries with key == v belong to the top k
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d));
  return v;
}

// Smallest and largest order key in cs[0..cnt).
__device__ __forceinline__ void wave_key_range(const float* cs, int cnt, uint32_t& lo, uint32_t& hi) {
  uint32_t a = 0xFFFFFFFFu, b = 0u;
  for (int i = lane_id(); i < cnt; i += kWave) {
    const uint32_t key = order_key(cs[i]);
    a = min(a, key);
    b = max(b, key);
  }
  lo = wave_min_u32(a);
  hi = wave_max_u32(b);
}

// Histogram of rel = key - lo over 256 bins (bin = (rel >> shift) & 255 for
// entries whose rel matches `prefix` above the digit) and the bin holding the
// kk-th largest entry.  Returns the bin; `above` = entries in higher bins,
// `in_bin` = entries in the bin.
__device__ int wave_hist_pick(const float* cs, int cnt, uint32_t lo, int shift, uint32_t pmask,
                              uint32_t prefix, int kk, uint32_t* hist, int& above, int& in_bin) {
  const int l = lane_id();
  *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
  wave_lds_sync();
  for (int i = l; i < cnt; i += kWave) {
    const uint32_t rel = order_key(cs[i]) - lo;
    if ((rel & pmask) == prefix) atomicAdd(&hist[(rel >> shift) & 255u], 1u);
  }
  wave_lds_sync();
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

__device__ __forceinline__ int range_bits8(uint32_t range) {   // bit length rounded up to 8
  const int nbits = range == 0u ? 0 : 32 - __clz((int)range);
  return (nbits + 7) & ~7;
}

// Exact k-th best among cs[0..cnt) (cnt >= k >= 1): radix select on the key
// offsets from the buffer minimum, 8 bits per pass from the top of the range.
__device__ Thresh wave_select_kth(const float* cs, int cnt, int k, uint32_t* hist) {
  uint32_t lo, hi;
  wave_key_range(cs, cnt, lo, hi);
  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  for (int shift = range_bits8(hi - lo) - 8; shift >= 0; shift -= 8) {
    int above, in_bin;
    const int b = wave_hist_pick(cs, cnt, lo, shift, pmask, prefix, kk, hist, above, in_bin);
    kk -= above;
    prefix |= (uint32_t)b << shift;
    pmask |= 0xFFu << shift;
  }
  return Thresh{lo + prefix, kk};
}

// Stable in-place compaction: keeps entries with key > t.v and the first
// t.need entries with key == t.v (the lowest positions, since the buffer is
// in ascending position order).  Returns the new count.
__device__ int wave_compact(float* cs, int* cp, int cnt, Thresh t) {
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  for (int base = 0; base < cnt; base += kWave) {
    const int i = base + l;
    const bool in = i < cnt;
    const float sc = in ? cs[i] : 0.0f;
    const int ps = in ? cp[i] : 0;
    const uint32_t key = order_key(sc);
    const bool eq = in && key == t.v;
    const uint64_t em = __ballot(eq);
    const bool keep = (in && key > t.v) || (eq && eq_seen + wave_prefix(em) < t.need);
    const uint64_t km = __ballot(keep);
    wave_lds_sync();   // this chunk is in registers before anything is overwritten
    if (keep) {
      const int o = out + wave_prefix(km);
      cs[o] = sc;
      cp[o] = ps;
    }
    out += __popcll(km);
    eq_seen += __popcll(em);
  }
  wave_lds_sync();
  return out;
}

// Buffer compaction during the stream, in the score-value domain.  One
// histogram over [lo, hi] (lo: a lower bound of every entry, hi: the largest
// entry) gives the bin b holding the k-th best; every entry in bins >= b is
// kept.  The bin map is monotone in the score, so the kept set is {s >= s*}
// with at least k members: the k-th best is >= s*, nothing below s* can win,
// and a later key equal to s* loses the position tie, so tau = s* keeps the
// strict filter exact.  A crowded bin (ties, or a range too wide to split)
// falls back to the exact select.
__device__ void wave_shrink(float* cs, int* cp, int& cnt, float& tau, float hi, int k, int keep_max,
                            uint32_t* hist) {
  const int l = lane_id();
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) hi = fmaxf(hi, __shfl_xor(hi, dd));
  float lo = tau;
  if (lo == -INFINITY) {                       // first shrink: entries may be anything
    float a = INFINITY;
    for (int i = l; i < cnt; i += kWave) a = fminf(a, cs[i]);
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) a = fminf(a, __shfl_xor(a, dd));
    lo = a;
  }
  const float inv = 256.0f / (hi - lo);
  if (hi > lo && inv > 0.0f && inv < INFINITY) {
    *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
    for (int i = l; i < cnt; i += kWave) {
      const int bin = min(255, max(0, (int)((cs[i] - lo) * inv)));
      atomicAdd(&hist[bin], 1u);
    }
    wave_lds_sync();
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const uint32_t tot = h.x + h.y + h.z + h.w;
    const int a3 = (int)(wave_suffix_sum(tot) - tot);
    const int a2 = a3 + (int)h.w, a1 = a2 + (int)h.z, a0 = a1 + (int)h.y;
    int bin = -1, kept = 0;
    if (a3 < k && k <= a2) { bin = 4 * l + 3; kept = a2; }
    else if (a2 < k && k <= a1) { bin = 4 * l + 2; kept = a1; }
    else if (a1 < k && k <= a0) { bin = 4 * l + 1; kept = a0; }
    else if (a0 < k && k <= a0 + (int)h.x) { bin = 4 * l; kept = a0 + (int)h.x; }
    const uint64_t mb = __ballot(bin >= 0);
    const int src = __ffsll((unsigned long long)mb) - 1;
    const int b = __shfl(bin, src);
    if (__shfl(kept, src) <= keep_max) {
      int out = 0;
      float smin = INFINITY;
      for (int base = 0; base < cnt; base += kWave) {
        const int i = base + l;
        const bool in = i < cnt;
        const float sc = in ? cs[i] : 0.0f;
        const int ps = in ? cp[i] : 0;
        const bool keep = in && min(255, max(0, (int)((sc - lo) * inv))) >= b;
        const uint64_t km = __ballot(keep);
        wave_lds_sync();
        if (keep) {
          const int o = out + wave_prefix(km);
          cs[o] = sc;
          cp[o] = ps;
          smin = fminf(smin, sc);
        }
        out += __popcll(km);
      }
#pragma unroll
      for (int dd = 32; dd >= 1; dd >>= 1) smin = fminf(smin, __shfl_xor(smin, dd));
      wave_lds_sync();
      cnt = out;
      tau = smin;
      return;
    }
  }
  const Thresh th = wave_select_kth(cs, cnt, k, hist);
  cnt = wave_compact(cs, cp, cnt, th);
  tau = key_value(th.v);
}

// Same selection as wave_compact, but writes the kept positions to `dst`.
__device__ void wave_emit(const float* cs, const int* cp, int cnt, Thresh t, int32_t* dst) {
  const int l = lane_id();
  int out = 0, eq_seen = 0;
  for (int base = 0; base < cnt; base += kWave) {
    const int i = base + l;
    const bool in = i < cnt;
    const uint32_t key = order_key(in ? cs[i] : 0.0f);
    const bool eq = in && key == t.v;
    const uint64_t em = __ballot(eq);
    const bool keep = (in && key > t.v) || (eq && eq_seen + wave_prefix(em) < t.need);
    const uint64_t km = __ballot(keep);
    if (keep) dst[out + wave_prefix(km)] = cp[i];
    out += __popcll(km);
    eq_seen += __popcll(em);
  }
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

constexpr int kRing = 3;   // LDS tile buffers: tiles it, it+1 ready/landing, it+2 loading

// One half-tile block: the MFMAs of key half `nt` of the current tile into
// acc_mma and/or the epilogue of the other accumulator half (acc_epi), in one
// basic block so the scheduler can put the VALU work between MFMAs.  Returns
// the partial (this lane's 16 x HT heads) score of the epilogue half.
template <int HT, int KS, bool MMA, bool EPI>
__device__ __forceinline__ float half_block(const bf16x8 (&qf)[HT][KS], const float (&wr)[HT][16],
                                            const bf16x8 (&bfr)[KS], f32x16 (&acc_mma)[HT],
                                            const f32x16 (&acc_epi)[HT]) {
  if constexpr (MMA) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        acc_mma[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][ks], bfr[ks],
                                                              ks == 0 ? f32x16{} : acc_mma[ht], 0, 0, 0);
  }
  float part = 0.0f;
  if constexpr (EPI) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};     // 4 independent chains
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r & 3] = fmaf(wr[ht][r], fmaxf(acc_epi[ht][r], 0.0f), s[r & 3]);
    part = (s[0] + s[1]) + (s[2] + s[3]);
  }
  if constexpr (MMA && EPI) {
#pragma unroll
    for (int i = 0; i < HT * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                          // 4 VALU
    }
  }
  return part;
}

template <int KS>
__device__ __forceinline__ void read_bfrags(const unsigned char* kb, int nt, int m, int hf, bf16x8 (&bfr)[KS]) {
  using G = TileGeom<KS>;
  const int r = nt * 32 + m;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    bfr[ks] = *reinterpret_cast<const bf16x8*>(kb + r * G::row_bytes + G::swz(r, hf * (G::CPR / 2) + ks) * 16);
}

template <int HT, int KS, bool SCALE>
__global__ __launch_bounds__(kThreads, 1) void fused_indexer_topk_kernel(FusedArgs a) {
  using G = TileGeom<KS>;
  constexpr int d = G::d;
  constexpr int kLoads = G::inst_per_wave + (SCALE ? 1 : 0);   // direct loads per wave per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* key_lds0 = smem;                                                   // [3][tile]
  float* scale_lds = reinterpret_cast<float*>(smem + kRing * G::tile_bytes);       // [3][64]
  int* need_flags = reinterpret_cast<int*>(scale_lds + kRing * kTileKeys);         // [2][4]
  uint32_t* hist = reinterpret_cast<uint32_t*>(need_flags + 8);                    // [4][256]
  float* cand = reinterpret_cast<float*>(hist + kRowsPerWG * 256);                 // [4][2C]

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m = l & 31, hf = l >> 5;
  const int b = blockIdx.y;
  const int row0 = (gridDim.x - 1 - blockIdx.x) * kRowsPerWG;
  const int t = row0 + wave;
  const bool row_ok = t < a.n_q;
  const int p = (int)a.q_start + (row_ok ? t : 0);              // positions fit in int32
  const int last_row = min(row0 + kRowsPerWG - 1, a.n_q - 1);
  const int n_keys = (int)a.q_start + last_row + 1;
  const int n_tiles = (n_keys + kTileKeys - 1) / kTileKeys;
  const int C = a.C;
  float* cs = cand + (size_t)wave * 2 * C;
  int* cp = reinterpret_cast<int*>(cs + C);
  uint32_t* my_hist = hist + wave * 256;

  // Query slice (A operand): lane (m, hf) holds head ht*32+m, elements
  // [hf*d/2 + 8*ks, +8) of d for k-step ks.  The key B operand uses the same
  // element split, so each dot product runs over all d elements.
  bf16x8 qf[HT][KS];
  float wr[HT][16];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_q + (row_ok ? t : 0)) * a.H * d;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + m;
      const bool ok = row_ok && h < a.H;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ht][ks] = ok ? *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * d + hf * (d / 2) + 8 * ks)
                        : bf16x8{};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hh = ht * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);   // MFMA output row of acc[r]
        wr[ht][r] = (row_ok && hh < a.H) ? a.w[((int64_t)b * a.n_q + t) * a.H + hh] : 0.0f;
      }
    }
  }

  const uint16_t* keys_b = a.keys + (int64_t)b * a.key_bstride;
  const float* scale_b = SCALE ? a.scale + (int64_t)b * a.scale_bstride : nullptr;

  // Direct HBM -> LDS loads of tile `it` into ring slot `slot`: load j of this
  // wave fills LDS slots [64J, 64J+64) (J = wave + 4j) in lane order, so lane l
  // fetches the global chunk that belongs in slot 64J + l.  Rows past the last
  // key are clamped (their scores are masked).
  auto issue_tile = [&](int it, int slot) {
    const int s0 = it * kTileKeys;
    unsigned char* tb = key_lds0 + slot * G::tile_bytes;
#pragma unroll
    for (int j = 0; j < G::inst_per_wave; ++j) {
      const int J = wave + 4 * j;
      const int S = J * G::lanes_per_inst + l;                 // LDS slot this lane fills
      const int r = S / G::CPR, sl = S % G::CPR;
      const int c = G::swz(r, sl);                             // swz is an involution
      const uint16_t* src = keys_b + (int64_t)min(s0 + r, n_keys - 1) * d + c * 8;
      if (G::lanes_per_inst == 64 || l < G::lanes_per_inst)
        __builtin_amdgcn_global_load_lds((void*)src, (lds_ptr_t)(tb + J * G::lanes_per_inst * 16), 16, 0, 0);
    }
    if constexpr (SCALE) {
      const float* src = scale_b + min(s0 + 16 * wave + (l & 15), n_keys - 1);
      if (l < 16)
        __builtin_amdgcn_global_load_lds((void*)src, (lds_ptr_t)(scale_lds + slot * kTileKeys + 16 * wave), 4, 0, 0);
    }
  };

  float tau = -INFINITY, vmax = -INFINITY;
  int cnt = 0;
  const int keep_max = C - 2 * kWave;          // after a shrink the next trigger is >= 64 appends away
  float sc_prev = 1.0f;
  float part0 = 0.0f;                           // nt=0 partial score of the tile being finished

  issue_tile(0, 0);
  if (n_tiles > 1) {
    issue_tile(1, 1);
    wait_vmcnt<kLoads>();
  } else {
    wait_vmcnt<0>();
  }
  if (tid < 8) need_flags[tid] = 0;
  __syncthreads();

  f32x16 acc0[HT], acc1[HT];
  int slot = 0;                                  // ring slot of tile it
  for (int it = 0; it <= n_tiles; ++it) {
    const bool mma = row_ok && it < n_tiles && it * kTileKeys <= p;
    const bool epi = row_ok && it >= 1 && (it - 1) * kTileKeys <= p;
    const unsigned char* kb = key_lds0 + slot * G::tile_bytes;
    const float sc_cur = SCALE ? scale_lds[slot * kTileKeys + l] : 1.0f;
    const u32x4 nf = *reinterpret_cast<const u32x4*>(need_flags + ((it & 1) ^ 1) * 4);   // previous step's
    const bool more = it + 2 < n_tiles;
    if (more) issue_tile(it + 2, slot == 0 ? 2 : slot - 1);   // (slot + 2) % 3

    bf16x8 bx[KS], by[KS];
    if (mma) {
      read_bfrags<KS>(kb, 0, m, hf, bx);
      read_bfrags<KS>(kb, 1, m, hf, by);
    }
    // block X: MFMAs of half 0 of tile it || epilogue of half 1 of tile it-1
    float part1 = 0.0f;
    if (mma && epi) part1 = half_block<HT, KS, true, true>(qf, wr, bx, acc0, acc1);
    else if (mma) half_block<HT, KS, true, false>(qf, wr, bx, acc0, acc1);
    else if (epi) part1 = half_block<HT, KS, false, true>(qf, wr, bx, acc0, acc1);

    if (epi) {
      // finish tile it-1: lanes 0-31 take key half 0, lanes 32-63 half 1
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part0), __float_as_uint(part1),
                                                       false, false);
      float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (SCALE) score *= sc_prev;
      const int s = (it - 1) * kTileKeys + l;
      if (s > p) score = -INFINITY;
      if ((nf.x | nf.y | nf.z | nf.w) && cnt > a.k + (C - a.k) / 2) {   // some row is nearly full
        wave_lds_sync();
        wave_shrink(cs, cp, cnt, tau, vmax, a.k, keep_max, my_hist);
      }
      const bool pass = score > tau;
      const uint64_t pm = __ballot(pass);
      if (pm) {
        if (pass) {
          const int o = cnt + wave_prefix(pm);
          cs[o] = score;
          cp[o] = s;
        }
        cnt += __popcll(pm);
        if (pass) vmax = fmaxf(vmax, score);      // per lane; reduced when a shrink needs it
      }
    }
    // block Y: MFMAs of half 1 of tile it || epilogue of its half 0
    if (mma) part0 = half_block<HT, KS, true, true>(qf, wr, by, acc1, acc0);
    sc_prev = sc_cur;
    if (l == 0) need_flags[(it & 1) * 4 + wave] = (row_ok && cnt > C - kWave) ? 1 : 0;
    if (more) wait_vmcnt<kLoads>();              // tile it+1 landed (it+2 may still fly)
    else wait_vmcnt<0>();
    __syncthreads();
    slot = slot == 2 ? 0 : slot + 1;
  }

  if (row_ok) {
    int32_t* dst = a.idx + ((int64_t)b * a.n_q + t) * a.k;
    wave_lds_sync();
    int written;
    if (cnt > a.k) {
      const Thresh th = wave_select_kth(cs, cnt, a.k, my_hist);
      wave_emit(cs, cp, cnt, th, dst);
      written = a.k;
    } else {
      for (int i = l; i < cnt; i += kWave) dst[i] = cp[i];
      written = cnt;
    }
    for (int i = written + l; i < a.k; i += kWave) dst[i] = -1;
  }
}

__global__ void upcast_fp8_kernel(const uint8_t* __restrict__ src, int64_t src_bstride,
                                  uint16_t* __restrict__ dst, int64_t dst_bstride,
                                  int64_t chunks_per_seq, int64_t total_chunks) {
  // one 16-code chunk per thread per step; d % 16 == 0 keeps chunks inside rows
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = c / chunks_per_seq, off = (c % chunks_per_seq) * 16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + b * src_bstride + off);
    u32x4 o0, o1;
    u32x2 r;
    r = e4m3x4_to_bf16x4(v.x); o0.x = r.x; o0.y = r.y;
    r = e4m3x4_to_bf16x4(v.y); o0.z = r.x; o0.w = r.y;
    r = e4m3x4_to_bf16x4(v.z); o1.x = r.x; o1.y = r.y;
    r = e4m3x4_to_bf16x4(v.w); o1.z = r.x; o1.w = r.y;
    u32x4* dd = reinterpret_cast<u32x4*>(dst + b * dst_bstride + off);
    dd[0] = o0;
    dd[1] = o1;
  }
}

template <int HT, int KS, bool SCALE>
hipError_t launch_fused_s(const FusedArgs& a, int B, hipStream_t s) {
  const size_t lds = fused_lds_bytes(KS * 16, a.C);
  const void* fn = reinterpret_cast<const void*>(&fused_indexer_topk_kernel<HT, KS, SCALE>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((a.n_q + kRowsPerWG - 1) / kRowsPerWG, B);
  hipLaunchKernelGGL((fused_indexer_topk_kernel<HT, KS, SCALE>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int HT, int KS>
hipError_t launch_fused_t(const FusedArgs& a, int B, hipStream_t s) {
  return a.scale ? launch_fused_s<HT, KS, true>(a, B, s) : launch_fused_s<HT, KS, false>(a, B, s);
}

}  // namespace

int fused_candidates(int k) {
  int extra = k / 2 > 2 * kWave ? k / 2 : 2 * kWave;
  return ((k + extra + kWave - 1) / kWave) * kWave;
}

size_t fused_lds_bytes(int d, int C) {
  const size_t tile = (size_t)kTileKeys * 2 * d;
  return kRing * tile + kRing * kTileKeys * sizeof(float) + 8 * sizeof(int) +
         kRowsPerWG * 256 * sizeof(uint32_t) + (size_t)kRowsPerWG * C * 8;
}

bool fused_dim_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

hipError_t launch_fused_indexer(const FusedArgs& a, int B, int d, hipStream_t s) {
  const int HT = a.H > 32 ? 2 : 1;
  const int KS = d / 16;
#define IX_FUSED_CASE(ht, ks) \
  if (HT == ht && KS == ks) return launch_fused_t<ht, ks>(a, B, s);
  IX_FUSED_CASE(1, 1) IX_FUSED_CASE(1, 2) IX_FUSED_CASE(1, 4) IX_FUSED_CASE(1, 8)
  IX_FUSED_CASE(2, 1) IX_FUSED_CASE(2, 2) IX_FUSED_CASE(2, 4) IX_FUSED_CASE(2, 8)
#undef IX_FUSED_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_upcast_fp8(const uint8_t* src, int64_t src_bstride, uint16_t* dst,
                             int64_t dst_bstride, int B, int64_t rows, int d, hipStream_t s) {
  const int64_t per_seq = rows * d / 16;
  const int64_t total = per_seq * B;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(upcast_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, src_bstride,
                     dst, dst_bstride, per_seq, total);
  return hipGetLastError();
}

}  // namespace ix
