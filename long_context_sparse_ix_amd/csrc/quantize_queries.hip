// Indexer queries into the fp8 form the declared fp8-query indexer reads.
//
// The indexer is a small FP8 module (IndexCache notes, section 1); a caller
// that declares fp8 queries passes e4m3fn codes with one fp32 scale per
// (row, head).  This kernel makes them from bf16 query rows with the key
// cache's per-row scaling (the library's reading; the pages give none):
// scale = max_j |q_j| / 448, or 1 for an all-zero row, and code_j =
// e4m3fn(q_j / scale), rounded to nearest with ties to the even code and
// saturating at +-448; both divisions are correctly rounded fp32.  A row is
// one (query row, head) of d values: G lanes hold 8 values each (G = d / 8
// rounded up to a power of two), so one wave encodes 64 / G rows per pass,
// the row maximum is a G-lane butterfly, and every lane reads 16 bytes and
// writes 8.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ix {

namespace {

constexpr int kWavesPerWG = 4;

template <int G>
__global__ __launch_bounds__(kWavesPerWG * kWave) void quantize_queries_kernel(const uint16_t* __restrict__ src,
                                                                                 uint8_t* __restrict__ codes,
                                                                                 float* __restrict__ scale,
                                                                                 int64_t n_rows, int dim) {
  constexpr int R = kWave / G;                       // rows per wave and pass
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int sub = l % G, grp = l / G;
  const bool col_ok = 8 * sub < dim;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerWG * R;
  for (int64_t base = ((int64_t)blockIdx.x * kWavesPerWG + wave) * R; base < n_rows; base += stride) {
    const int64_t row = base + grp;
    const bool ok = col_ok && row < n_rows;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(src + row * dim + 8 * sub);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(v[i] << 16);
      x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));   // within the row's G lanes
    const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
    if (ok) {
      uint32_t c[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i >> 2] |= e4m3fn_code(__fdiv_rn(x[i], s)) << (8 * (i & 3));
      *reinterpret_cast<u32x2*>(codes + row * dim + 8 * sub) = u32x2{c[0], c[1]};
    }
    if (sub == 0 && row < n_rows) scale[row] = s;
  }
}

template <int G>
hipError_t launch_g(const uint16_t* src, uint8_t* codes, float* scale, int64_t n_rows, int dim, hipStream_t s) {
  constexpr int rows_per_wg = kWavesPerWG * (kWave / G);
  int64_t blocks = (n_rows + rows_per_wg - 1) / rows_per_wg;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_queries_kernel<G>, dim3((unsigned)blocks), dim3(kWavesPerWG * kWave), 0, s, src,
                     codes, scale, n_rows, dim);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_queries(const uint16_t* src, uint8_t* codes, float* scale, int64_t n_rows, int dim,
                                   hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int lanes = dim / 8;
  if (lanes <= 2) return launch_g<2>(src, codes, scale, n_rows, dim, s);
  if (lanes <= 4) return launch_g<4>(src, codes, scale, n_rows, dim, s);
  if (lanes <= 8) return launch_g<8>(src, codes, scale, n_rows, dim, s);
  if (lanes <= 16) return launch_g<16>(src, codes, scale, n_rows, dim, s);
  return hipErrorInvalidValue;
}

}  // namespace ix
