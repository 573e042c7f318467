// Per-row overlap of two index buffers.
//
// Reuse of one layer's positions by the next layers works because adjacent
// layers' top-k sets overlap heavily ("IndexShare", LLM Architecture Gallery,
// section "Why Reusing Indices Can Work"); this counts, for every query row,
// the positions present in both rows.  One wave per row: row b goes to LDS,
// then each lane binary-searches its share of row a's valid positions among
// row b's valid prefix.  Rows are in the layout the indexer writes (ascending
// valid positions, then -1); for any other layout every access still stays
// inside the row.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kRowsPerWG = 4;

__global__ __launch_bounds__(kRowsPerWG * kWave) void index_overlap_kernel(const int32_t* __restrict__ a,
                                                                           const int32_t* __restrict__ b,
                                                                           int32_t* __restrict__ counts,
                                                                           int64_t rows, int k) {
  extern __shared__ int32_t sb[];                // [kRowsPerWG][k]
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + wave;
  if (row >= rows) return;                        // wave-level only: no workgroup barrier below
  int32_t* mb = sb + wave * k;
  const int32_t* arow = a + row * k;
  const int32_t* brow = b + row * k;
  int nb = 0;
  for (int i = l; i < k; i += kWave) {
    const int32_t v = brow[i];
    mb[i] = v;
    nb += v >= 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) nb += __shfl_xor(nb, d);
  wave_lds_sync();
  int c = 0;
  for (int i = l; i < k; i += kWave) {
    const int32_t x = arow[i];
    if (x < 0) continue;
    int lo = 0, hi = nb;                          // first slot with value >= x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (mb[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    c += (lo < nb && mb[lo] == x) ? 1 : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
  if (l == 0) counts[row] = c;
}

}  // namespace

hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int32_t* counts, int64_t rows, int k,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const size_t lds = (size_t)kRowsPerWG * k * sizeof(int32_t);
  hipLaunchKernelGGL(index_overlap_kernel, dim3((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG)),
                     dim3(kRowsPerWG * kWave), lds, s, a, b, counts, rows, k);
  return hipGetLastError();
}

}  // namespace ix
