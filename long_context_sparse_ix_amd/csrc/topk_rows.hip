// Per-row top-k over materialised fp32 score rows.
//
// Selection rule ("IndexShare", LLM Architecture Gallery, section "How
// IndexShare Works": the full layer performs the top-k operation and stores the
// selected positions): keep the min(k, p+1) best positions of row p under
// (score desc, position asc); emit them in ascending position order, then -1.
//
// One 1024-thread workgroup per row.  Four 8-bit radix passes over the row's
// order keys (LDS histogram) find the exact k-th key v and how many ties at v
// are needed; a final pass in position order keeps key > v and the first ties
// at v, with block-wide prefix sums giving each kept position its output slot.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void topk_rows_kernel(const float* __restrict__ scores,
                                                             int64_t ld, int32_t* __restrict__ idx,
                                                             int n_q, int64_t q_start, int k) {
  __shared__ uint32_t hist[256];
  __shared__ int sel_bin, sel_above;
  __shared__ int wave_keep[kWaves], wave_eq[kWaves];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int row = blockIdx.x;
  const int t = row % n_q;
  const int64_t n = q_start + t + 1;
  const float* src = scores + (int64_t)row * ld;
  int32_t* dst = idx + (int64_t)row * k;

  if (n <= k) {
    for (int64_t i = tid; i < k; i += kThreads) dst[i] = i < n ? (int32_t)i : -1;
    return;
  }

  uint32_t prefix = 0u, pmask = 0u;
  int kk = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kThreads) {
      const uint32_t key = order_key(src[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
      const uint32_t tot = h0 + h1 + h2 + h3;
      const int a3 = (int)(wave_suffix_sum(tot) - tot);
      const int a2 = a3 + (int)h3, a1 = a2 + (int)h2, a0 = a1 + (int)h1;
      int bin = -1, above = 0;
      if (a3 < kk && kk <= a2) { bin = 4 * l + 3; above = a3; }
      else if (a2 < kk && kk <= a1) { bin = 4 * l + 2; above = a2; }
      else if (a1 < kk && kk <= a0) { bin = 4 * l + 1; above = a1; }
      else if (a0 < kk && kk <= a0 + (int)h0) { bin = 4 * l; above = a0; }
      if (bin >= 0) { sel_bin = bin; sel_above = above; }
    }
    __syncthreads();
    kk -= sel_above;
    prefix |= (uint32_t)sel_bin << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t v = prefix;
  const int need = kk;

  int out_base = 0, eq_base = 0;
  for (int64_t base = 0; base < n; base += kThreads) {
    const int64_t i = base + tid;
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
    if (keep) dst[keep_before + wave_prefix(km)] = (int32_t)i;
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
