// Per-row overlap of two index buffers.
//
// Reuse of one layer's positions by the next layers works because adjacent
// layers' top-k sets overlap heavily ("IndexShare", LLM Architecture Gallery,
// section "Why Reusing Indices Can Work"); this counts, for every query row,
// the positions present in both rows.  One wave per row: row b goes to LDS;
// lane l holds row a's slots [C l, C l + C) in registers (C = k / 64 rounded
// up), finds its first valid position's place in row b's valid prefix by one
// binary search, and then walks row b alongside its slots, as a merge of two
// ascending lists: about C + log2(k) + (row b's entries in the lane's range)
// LDS reads per lane instead of a binary search per position.  Rows are in
// the layout the indexer writes (ascending valid positions, then -1); for any
// other layout the count is unspecified, but every access stays inside the
// row and every walk ends (its index only moves forward).
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kRowsPerWG = 4;
constexpr int kMaxChunk = 32;             // row a's slots per lane: k <= 2048

__global__ __launch_bounds__(kRowsPerWG * kWave) void index_overlap_kernel(const int32_t* __restrict__ a,
                                                                           const int32_t* __restrict__ b,
                                                                           int32_t* __restrict__ counts,
                                                                           int64_t rows, int k) {
  extern __shared__ __align__(16) int32_t sb[];   // [kRowsPerWG][k]
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + wave;
  if (row >= rows) return;                        // wave-level only: no workgroup barrier below
  int32_t* mb = sb + wave * k;
  const int32_t* arow = a + row * k;
  const int32_t* brow = b + row * k;
  // this lane's slots of row a, all loads issued before row b's: 16 bytes
  // a load when k and C are multiples of 4 (the rows and every lane's first
  // slot then sit on 16-byte boundaries; the buffers are 16-byte aligned)
  const int C = (k + kWave - 1) / kWave;
  const int c0 = l * C;
  const bool vec = (k & 3) == 0 && (C & 3) == 0;
  int32_t av[kMaxChunk];
  if (vec) {
#pragma unroll
    for (int j = 0; j < kMaxChunk; j += 4) {
      u32x4 q = {~0u, ~0u, ~0u, ~0u};
      if (j < C && c0 + j < k) q = *reinterpret_cast<const u32x4*>(arow + c0 + j);   // c0 + j < k and k % 4 == 0: all four inside
      av[j] = (int32_t)q.x; av[j + 1] = (int32_t)q.y; av[j + 2] = (int32_t)q.z; av[j + 3] = (int32_t)q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxChunk; ++j) av[j] = (j < C && c0 + j < k) ? arow[c0 + j] : -1;
  }
  int nb = 0;
  if (vec) {
    for (int i = 4 * l; i < k; i += 4 * kWave) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(brow + i);
      *reinterpret_cast<u32x4*>(mb + i) = v;
      nb += ((int32_t)v.x >= 0) + ((int32_t)v.y >= 0) + ((int32_t)v.z >= 0) + ((int32_t)v.w >= 0);
    }
  } else {
    for (int i = l; i < k; i += kWave) {
      const int32_t v = brow[i];
      mb[i] = v;
      nb += v >= 0;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) nb += __shfl_xor(nb, d);
  wave_lds_sync();
  int c = 0, p = -1;                              // p: next slot of row b to compare
#pragma unroll
  for (int j = 0; j < kMaxChunk; ++j) {
    const int32_t x = av[j];
    if (x < 0) continue;
    if (p < 0) {                                  // first valid position: its place in row b
      int lo = 0, hi = nb;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (mb[mid] < x) lo = mid + 1;
        else hi = mid;
      }
      p = lo;
    }
    int32_t y = p < nb ? mb[p] : INT32_MAX;
    while (y < x) {
      ++p;
      y = p < nb ? mb[p] : INT32_MAX;
    }
    if (y == x) {
      ++c;
      ++p;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
  if (l == 0) counts[row] = c;
}

}  // namespace

hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int32_t* counts, int64_t rows, int k,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > kMaxChunk * kWave) return hipErrorInvalidValue;
  const size_t lds = (size_t)kRowsPerWG * k * sizeof(int32_t);
  hipLaunchKernelGGL(index_overlap_kernel, dim3((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG)),
                     dim3(kRowsPerWG * kWave), lds, s, a, b, counts, rows, k);
  return hipGetLastError();
}

}  // namespace ix
