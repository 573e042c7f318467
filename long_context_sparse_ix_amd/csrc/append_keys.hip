// New indexer keys into the fp8 key cache.
//
// The indexer keys are stored in FP8 (IndexCache notes, section 1, which
// describes the indexer as a small, low-rank, FP8 module).  Per-row scaling (the library's reading; the pages
// give none): scale = max_j |k_j| / 448, or 1 for an all-zero row, and
// code_j = e4m3fn(k_j / scale), rounded to nearest with ties to the even code
// and saturating at +-448; both divisions are correctly rounded fp32.  One
// wave per new row; every lane encodes two neighbouring elements in software
// (exact power-of-two rescaling and rintf), so the codes do not depend on a
// conversion instruction's rounding or saturation mode.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kRowsPerWG = 4;

__global__ __launch_bounds__(kRowsPerWG * kWave) void append_keys_kernel(const float* __restrict__ k_new,
                                                                         uint8_t* __restrict__ k_cache,
                                                                         float* __restrict__ k_scale, int n_new,
                                                                         int64_t rows, int64_t pos,
                                                                         const int64_t* __restrict__ seq_shift,
                                                                         int64_t shift_bound, int64_t kv_cap, int dim) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + wave;   // b * n_new + r
  if (row >= rows) return;
  const int64_t b = row / n_new, r = row % n_new;
  const bool on = 2 * l < dim;
  float2 x = make_float2(0.0f, 0.0f);
  if (on) x = *reinterpret_cast<const float2*>(k_new + row * dim + 2 * l);
  float amax = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
  const float scale = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
  // per-sequence rows: shifted back by the sequence's distance below the bound
  const int64_t pos_b = seq_shift ? pos - shift_bound + seq_start(seq_shift, (int)b, shift_bound) : pos;
  const int64_t dst = b * kv_cap + pos_b + r;
  if (on) {
    const uint32_t c0 = e4m3fn_code(__fdiv_rn(x.x, scale));
    const uint32_t c1 = e4m3fn_code(__fdiv_rn(x.y, scale));
    *reinterpret_cast<uint16_t*>(k_cache + dst * dim + 2 * l) = (uint16_t)(c0 | (c1 << 8));
  }
  if (l == 0) k_scale[dst] = scale;
}

}  // namespace

hipError_t launch_append_keys(const float* k_new, uint8_t* k_cache, float* k_scale, int B, int n_new, int64_t pos,
                              const int64_t* seq_shift, int64_t shift_bound, int64_t kv_cap, int dim,
                              hipStream_t s) {
  const int64_t rows = (int64_t)B * n_new;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(append_keys_kernel, dim3((unsigned)((rows + kRowsPerWG - 1) / kRowsPerWG)),
                     dim3(kRowsPerWG * kWave), 0, s, k_new, k_cache, k_scale, n_new, rows, pos, seq_shift,
                     shift_bound, kv_cap, dim);
  return hipGetLastError();
}

}  // namespace ix
