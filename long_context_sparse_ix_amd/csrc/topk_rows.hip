// Per-row top-k over materialised fp32 score rows.
//
// Selection rule ("IndexShare", LLM Architecture Gallery, section "How
// IndexShare Works": the full layer performs the top-k operation and stores the
// selected positions): keep the min(k, p+1) best positions of row p under
// (score desc, position asc); emit them in ascending position order, then -1.
//
// One 1024-thread workgroup per row, all passes over the row in L2:
//   1. min / max of the row (register reductions, no atomics);
//   2. a 2048-bin histogram over [min, max] in the value domain (LDS atomics
//      spread over the bins) gives the bin b holding the k-th best and the
//      number of entries above it;
//   3. an exact radix select on the order keys of bin b's entries only (8 bits
//      per pass over the bin's key range) finds the k-th key v and how many
//      ties at v are needed;
//   4. a stable pass in position order keeps key > v and the first ties at v,
//      with block-wide prefix sums giving each kept position its slot.
// The value-domain first pass keeps histogram contention low: a first pass on
// the top bits of the float key would put nearly every score in 2-3 bins.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;

__device__ __forceinline__ int vbin(float s, float lo, float inv) {
  return min(kBins - 1, max(0, (int)((s - lo) * inv)));
}

// Block-wide reductions through LDS scratch (one slot per wave).
__device__ __forceinline__ float block_min(float v, float* red) {
  for (int d = 32; d >= 1; d >>= 1) v = fminf(v, __shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kWaves; ++w) r = fminf(r, red[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Bin b of hist[0..nbins) with above(b) < kk <= above(b) + hist[b], where
// above(b) counts entries in bins > b.  Wave 0 scans; result via LDS.
__device__ void pick_from_top(const uint32_t* hist, int nbins, int kk, int* out_bin, int* out_above) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const int per = nbins / kWave;                 // consecutive bins per lane
    uint32_t tot = 0;
    for (int j = 0; j < per; ++j) tot += hist[l * per + j];
    const int above_lane = (int)(wave_suffix_sum(tot) - tot);
    if (above_lane < kk && kk <= above_lane + (int)tot) {     // exactly one lane
      int ab = above_lane;
      for (int j = per - 1; j >= 0; --j) {
        const int h = (int)hist[l * per + j];
        if (ab < kk && kk <= ab + h) {
          *out_bin = l * per + j;
          *out_above = ab;
          break;
        }
        ab += h;
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const float* __restrict__ scores,
                                                             int64_t ld, int32_t* __restrict__ idx,
                                                             int n_q, int64_t q_start, int k) {
  __shared__ uint32_t hist[kBins];
  __shared__ float red[kWaves];
  __shared__ int sel_bin, sel_above;
  __shared__ int wave_keep[kWaves], wave_eq[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int row = blockIdx.x;
  const int t = row % n_q;
  const int n = (int)(q_start + t + 1);
  const float* src = scores + (int64_t)row * ld;
  int32_t* dst = idx + (int64_t)row * k;

  if (n <= k) {
    for (int i = tid; i < k; i += kThreads) dst[i] = i < n ? i : -1;
    return;
  }

  // 1. range
  float a = INFINITY, b = -INFINITY;
  for (int i = tid; i < n; i += kThreads) {
    const float s = src[i];
    a = fminf(a, s);
    b = fmaxf(b, s);
  }
  const float lo = block_min(a, red);
  const float hi = block_max(b, red);

  // 2. value-domain histogram (skipped when all scores are equal or the
  //    range cannot be split: then every entry counts as bin 0)
  float inv = kBins / (hi - lo);
  if (!(hi > lo) || !(inv > 0.0f) || !(inv < INFINITY)) inv = 0.0f;
  for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) atomicAdd(&hist[vbin(src[i], lo, inv)], 1u);
  __syncthreads();
  pick_from_top(hist, kBins, k, &sel_bin, &sel_above);
  const int vb = sel_bin;
  int kk = k - sel_above;
  __syncthreads();

  // 3. exact radix select among bin vb's entries, on order-key offsets from
  //    the smallest key in the bin
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  {
    uint32_t a_min = 0xFFFFFFFFu, a_max = 0u;
    for (int i = tid; i < n; i += kThreads) {
      const float s = src[i];
      if (vbin(s, lo, inv) == vb) {
        const uint32_t key = order_key(s);
        a_min = min(a_min, key);
        a_max = max(a_max, key);
      }
    }
    for (int d = 32; d >= 1; d >>= 1) {
      a_min = min(a_min, (uint32_t)__shfl_xor((int)a_min, d));
      a_max = max(a_max, (uint32_t)__shfl_xor((int)a_max, d));
    }
    __shared__ uint32_t kred[2][kWaves];
    if (l == 0) {
      kred[0][wave] = a_min;
      kred[1][wave] = a_max;
    }
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      kmin = min(kmin, kred[0][w]);
      kmax = max(kmax, kred[1][w]);
    }
    __syncthreads();
  }
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0u ? 0 : 32 - __clz((int)range);
  uint32_t prefix = 0u, pmask = 0u;
  for (int shift = ((nbits + 7) & ~7) - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const float s = src[i];
      if (vbin(s, lo, inv) != vb) continue;
      const uint32_t rel = order_key(s) - kmin;
      if ((rel & pmask) == prefix) atomicAdd(&hist[(rel >> shift) & 255u], 1u);
    }
    __syncthreads();
    pick_from_top(hist, 256, kk, &sel_bin, &sel_above);
    kk -= sel_above;
    prefix |= (uint32_t)sel_bin << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t v = kmin + prefix;
  const int need = kk;

  // 4. stable emission in position order
  int out_base = 0, eq_base = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const bool in = i < n;
    const uint32_t key = in ? order_key(src[i]) : 0u;
    const bool eq = in && key == v;
    const uint64_t em = __ballot(eq);
    if (l == 0) wave_eq[wave] = __popcll(em);
    __syncthreads();
    int eq_before = eq_base;
    for (int w = 0; w < wave; ++w) eq_before += wave_eq[w];
    const bool keep = (in && key > v) || (eq && eq_before + wave_prefix(em) < need);
    const uint64_t km = __ballot(keep);
    if (l == 0) wave_keep[wave] = __popcll(km);
    __syncthreads();
    int keep_before = out_base;
    for (int w = 0; w < wave; ++w) keep_before += wave_keep[w];
    if (keep) dst[keep_before + wave_prefix(km)] = i;
    int kt = 0, et = 0;
    for (int w = 0; w < kWaves; ++w) { kt += wave_keep[w]; et += wave_eq[w]; }
    out_base += kt;
    eq_base += et;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk_rows(const float* scores, int64_t ld, int32_t* idx, int rows, int n_q,
                            int64_t q_start, int k, hipStream_t s) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(kThreads), 0, s, scores, ld, idx, n_q,
                     q_start, k);
  return hipGetLastError();
}

}  // namespace ix
