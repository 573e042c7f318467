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
//     barrier per tile) shared by the 4 rows;
//   * each wave keeps its row's 64 heads x d query slice in VGPRs as the MFMA
//     A operand (M = heads) and reads key tiles as the B operand (N = keys):
//     v_mfma_f32_32x32x16_bf16, output lane l holds key l%32 and 16 heads;
//   * epilogue: ReLU, head weight, sum over the lane's heads, then one
//     permlane32 swap + add finishes the head sum and leaves lane l holding the
//     score of key (tile start + l);
//   * streaming top-k per row: a strict "score > tau" filter appends survivors
//     to a wave-private LDS candidate buffer (kept in ascending position
//     order); when it nears capacity a wave-level radix select finds the
//     exact k-th best (score desc, position asc), a stable compaction keeps
//     exactly k, and tau becomes the k-th score.  Because keys arrive in
//     ascending position, a later key tying tau always loses the tie, so the
//     strict filter is exact.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kTileKeys = 64;
constexpr int kRowsPerWG = 4;
constexpr int kThreads = kRowsPerWG * kWave;

struct Thresh {
  uint32_t v;   // order key of the k-th best entry
  int need;     // how many entries with key == v belong to the top k
};

// Exact k-th best among cs[0..cnt) (wave-private LDS, cnt >= k >= 1) by a
// 4-pass, 8-bit radix select on the order keys.
__device__ Thresh wave_select_kth(const float* cs, int cnt, int k, uint32_t* hist) {
  const int l = lane_id();
  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
    for (int i = l; i < cnt; i += kWave) {
      const uint32_t key = order_key(cs[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    wave_lds_sync();
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const uint32_t tot = h.x + h.y + h.z + h.w;
    const int a3 = (int)(wave_suffix_sum(tot) - tot);   // entries in higher lanes' bins
    const int a2 = a3 + (int)h.w, a1 = a2 + (int)h.z, a0 = a1 + (int)h.y;
    int bin = -1, above = 0;
    if (a3 < kk && kk <= a2) { bin = 4 * l + 3; above = a3; }
    else if (a2 < kk && kk <= a1) { bin = 4 * l + 2; above = a2; }
    else if (a1 < kk && kk <= a0) { bin = 4 * l + 1; above = a1; }
    else if (a0 < kk && kk <= a0 + (int)h.x) { bin = 4 * l; above = a0; }
    const uint64_t m = __ballot(bin >= 0);
    const int src = __ffsll((unsigned long long)m) - 1;
    const int b = __shfl(bin, src);
    kk -= __shfl(above, src);
    prefix |= (uint32_t)b << shift;
    pmask |= 0xFFu << shift;
  }
  return Thresh{prefix, kk};
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

template <int KS>
struct TileGeom {
  static constexpr int d = KS * 16;
  static constexpr int row_bytes = 2 * d + 16;        // padded LDS row: conflict-free B reads
  static constexpr int tile_bytes = kTileKeys * row_bytes;
  static constexpr int chunks = kTileKeys * d / 8;    // 16-byte pieces per tile
  static constexpr int per_thread = (chunks + kThreads - 1) / kThreads;
};

template <int HT, int KS>
__global__ __launch_bounds__(kThreads, 1) void fused_indexer_topk_kernel(FusedArgs a) {
  using G = TileGeom<KS>;
  constexpr int d = G::d;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* key_lds0 = smem;
  float* scale_lds = reinterpret_cast<float*>(smem + 2 * G::tile_bytes);      // [2][64]
  uint32_t* hist = reinterpret_cast<uint32_t*>(scale_lds + 2 * kTileKeys);    // [4][256]

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m = l & 31, hf = l >> 5;
  const int b = blockIdx.y;
  const int row0 = (gridDim.x - 1 - blockIdx.x) * kRowsPerWG;
  const int t = row0 + wave;
  const bool row_ok = t < a.n_q;
  const int64_t p = a.q_start + (row_ok ? t : 0);
  const int last_row = min(row0 + kRowsPerWG - 1, a.n_q - 1);
  const int64_t n_keys = a.q_start + last_row + 1;
  const int n_tiles = (int)((n_keys + kTileKeys - 1) / kTileKeys);

  float* cs = reinterpret_cast<float*>(hist + kRowsPerWG * 256) + (size_t)wave * 2 * a.C;
  int* cp = reinterpret_cast<int*>(cs + a.C);
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
      for (int ks = 0; ks < KS; ++ks) {
        if (ok) {
          qf[ht][ks] = *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * d + hf * (d / 2) + 8 * ks);
        } else {
          qf[ht][ks] = bf16x8{};
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hh = ht * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);   // MFMA output row of acc[r]
        wr[ht][r] = (row_ok && hh < a.H) ? a.w[((int64_t)b * a.n_q + t) * a.H + hh] : 0.0f;
      }
    }
  }

  const uint16_t* keys_b = a.keys + (int64_t)b * a.key_bstride;
  const float* scale_b = a.scale ? a.scale + (int64_t)b * a.scale_bstride : nullptr;

  u32x4 pre[G::per_thread];
  float pre_scale = 1.0f;
  auto load_tile = [&](int it) {
    const int64_t s0 = (int64_t)it * kTileKeys;
#pragma unroll
    for (int j = 0; j < G::per_thread; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / (d / 8), col = c % (d / 8);
      if (c < G::chunks && s0 + r < n_keys) {
        pre[j] = *reinterpret_cast<const u32x4*>(keys_b + (s0 + r) * d + col * 8);
      } else {
        pre[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < kTileKeys) pre_scale = (scale_b && s0 + tid < n_keys) ? scale_b[s0 + tid] : 1.0f;
  };
  auto store_tile = [&](int buf) {
    unsigned char* dst = key_lds0 + buf * G::tile_bytes;
#pragma unroll
    for (int j = 0; j < G::per_thread; ++j) {
      const int c = tid + j * kThreads;
      const int r = c / (d / 8), col = c % (d / 8);
      if (c < G::chunks) *reinterpret_cast<u32x4*>(dst + r * G::row_bytes + col * 16) = pre[j];
    }
    if (tid < kTileKeys) scale_lds[buf * kTileKeys + tid] = pre_scale;
  };

  float tau = -INFINITY;
  int cnt = 0;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1);
    const int64_t s0 = (int64_t)it * kTileKeys;
    if (row_ok && s0 <= p) {
      const unsigned char* kb = key_lds0 + buf * G::tile_bytes;
      f32x16 acc[2][HT];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[nt][ht] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 bfr[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bfr[nt] = *reinterpret_cast<const bf16x8*>(kb + (nt * 32 + m) * G::row_bytes + hf * d + 16 * ks);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[nt][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][ks], bfr[nt], acc[nt][ht], 0, 0, 0);
      }
      float part[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float s = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int r = 0; r < 16; ++r) s = fmaf(wr[ht][r], fmaxf(acc[nt][ht][r], 0.0f), s);
        part[nt] = s;
      }
      // lanes 0-31: key tile 0 (own half + partner half); lanes 32-63: tile 1.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                       __float_as_uint(part[1]), false, false);
      float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      score *= scale_lds[buf * kTileKeys + l];
      const int64_t s = s0 + l;
      if (s > p) score = -INFINITY;
      const bool pass = score > tau;
      const uint64_t pm = __ballot(pass);
      if (pass) {
        const int o = cnt + wave_prefix(pm);
        cs[o] = score;
        cp[o] = (int)s;
      }
      cnt += __popcll(pm);
      if (cnt > a.C - kWave) {
        wave_lds_sync();
        const Thresh th = wave_select_kth(cs, cnt, a.k, my_hist);
        cnt = wave_compact(cs, cp, cnt, th);
        tau = key_value(th.v);
      }
    }
    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
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
    u32x4* d = reinterpret_cast<u32x4*>(dst + b * dst_bstride + off);
    d[0] = o0;
    d[1] = o1;
  }
}

template <int HT, int KS>
hipError_t launch_fused_t(const FusedArgs& a, int B, hipStream_t s) {
  const size_t lds = fused_lds_bytes(KS * 16, a.C);
  const void* fn = reinterpret_cast<const void*>(&fused_indexer_topk_kernel<HT, KS>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((a.n_q + kRowsPerWG - 1) / kRowsPerWG, B);
  hipLaunchKernelGGL((fused_indexer_topk_kernel<HT, KS>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int fused_candidates(int k) {
  int extra = k / 2 > kWave ? k / 2 : kWave;
  return ((k + extra + kWave - 1) / kWave) * kWave;
}

size_t fused_lds_bytes(int d, int C) {
  const size_t tile = (size_t)kTileKeys * (2 * d + 16);
  return 2 * tile + 2 * kTileKeys * sizeof(float) + kRowsPerWG * 256 * sizeof(uint32_t) +
         (size_t)kRowsPerWG * C * 8;
}

hipError_t launch_fused_indexer(const FusedArgs& a, int B, int d, hipStream_t s) {
  const int HT = a.H > 32 ? 2 : 1;
  const int KS = d / 16;
#define IX_FUSED_CASE(ht, ks) \
  if (HT == ht && KS == ks) return launch_fused_t<ht, ks>(a, B, s);
  IX_FUSED_CASE(1, 1) IX_FUSED_CASE(1, 2) IX_FUSED_CASE(1, 3) IX_FUSED_CASE(1, 4)
  IX_FUSED_CASE(1, 5) IX_FUSED_CASE(1, 6) IX_FUSED_CASE(1, 7) IX_FUSED_CASE(1, 8)
  IX_FUSED_CASE(2, 1) IX_FUSED_CASE(2, 2) IX_FUSED_CASE(2, 3) IX_FUSED_CASE(2, 4)
  IX_FUSED_CASE(2, 5) IX_FUSED_CASE(2, 6) IX_FUSED_CASE(2, 7) IX_FUSED_CASE(2, 8)
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
