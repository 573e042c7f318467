// Device-side helpers shared by the libix kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Completes this wave's outstanding LDS operations and stops the compiler
// from moving memory accesses across this point; used where lanes of one
// wave exchange data through LDS.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int wave_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Total order on fp32 scores as unsigned keys: a larger score gives a larger
// key; -0.0 is folded onto +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Four OCP e4m3fn codes (one dword) -> four bf16 values (two dwords).  Every
// e4m3fn value is exactly representable in bf16, so this is exact.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t codes) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Wave-wide inclusive prefix sum in lane order, in registers: DPP row_shr
// steps of 1, 2, 4 and 8 scan each 16-lane row (a lane whose source lies
// before its row adds the 0 given as the old value), then every row adds the
// totals of the rows before it, read from lanes 15, 31 and 47.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shr(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_shr<0x111>(v);     // row_shr:1
  v += dpp_shr<0x112>(v);     // row_shr:2
  v += dpp_shr<0x114>(v);     // row_shr:4
  v += dpp_shr<0x118>(v);     // row_shr:8
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  return v + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// Wave-wide inclusive suffix sum (lane l gets the sum over lanes >= l).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const uint32_t incl = wave_incl_scan(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1) - incl + v;
}

// Position of query row 0 of sequence b: the sequence's own start when a
// per-sequence array is given (clamped into [0, bound], so a bad entry can
// never move a read past the keys every launch is sized for), else the common
// start `bound`.
__device__ __forceinline__ int64_t seq_start(const int64_t* seq, int b, int64_t bound) {
  if (!seq) return bound;
  const int64_t v = seq[b];
  return v < 0 ? 0 : (v > bound ? bound : v);
}

// max(x, 0) as one v_med3_f32 (x clamped to [0, +inf]).  fmaxf would add a
// NaN-quieting max in front; the callers' inputs (MFMA dot products of finite
// bf16 values) are never NaN.
// e4m3fn (OCP FP8) code of y in software, |y| clamped to 448: round to
// nearest with ties to the even code; a negative value that rounds to zero
// keeps its sign bit, -0.0 and +0.0 give +0.  Exact power-of-two rescaling
// and one rintf, so the code does not depend on a conversion instruction's
// rounding or saturation mode.
constexpr float kE4M3Max = 448.0f;
__device__ __forceinline__ uint32_t e4m3fn_code(float y) {
  const uint32_t sign = y < 0.0f ? 0x80u : 0u;
  const float a = fminf(fabsf(y), kE4M3Max);
  if (a < 0.015625f) {                           // below the smallest normal 2^-6: m * 2^-9
    const uint32_t m = (uint32_t)rintf(a * 512.0f);   // exact scaling; m == 8 is the smallest normal
    return sign | m;
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;      // a is a normal fp32 here
  const float frac = ldexpf(a, -e);                              // exact, in [1, 2)
  uint32_t m = (uint32_t)rintf((frac - 1.0f) * 8.0f);            // exact operands, one rounding
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | m;
}

__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.402823466e38f); }

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask));
}

// op of v over lanes l and l ^ 16 (xor16_op) or l ^ 32 (xor32_op), in
// registers: with both operands v, v_permlane16_swap / v_permlane32_swap
// return v of the lane and of its partner (the last two steps of wave_reduce
// below).
template <typename Op>
__device__ __forceinline__ float xor16_op(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float xor32_op(float v, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Full-wave reduction with the result in every lane, in registers: DPP moves
// pair lanes within 16 (xor 1, xor 2, then the 8- and 16-lane mirrors, which
// pair each already-reduced half with the other), v_permlane16_swap and
// v_permlane32_swap the 16- and 32-lane halves (with both operands v, the two
// results hold v of the lane and of its partner).  __shfl_xor would take an
// LDS round trip (ds_bpermute) per step instead.  op must be associative and
// commutative (min, max, integer add).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  const auto bits = [](T x) { return __builtin_bit_cast(uint32_t, x); };
  const auto val = [](uint32_t x) { return __builtin_bit_cast(T, x); };
  v = op(v, val(dpp_mov<0xB1>(bits(v))));     // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, val(dpp_mov<0x4E>(bits(v))));     // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, val(dpp_mov<0x141>(bits(v))));    // row_half_mirror: 7 - i within 8
  v = op(v, val(dpp_mov<0x140>(bits(v))));    // row_mirror: 15 - i within 16
  auto r = __builtin_amdgcn_permlane16_swap(bits(v), bits(v), false, false);
  v = op(val(r[0]), val(r[1]));
  r = __builtin_amdgcn_permlane32_swap(bits(v), bits(v), false, false);
  return op(val(r[0]), val(r[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float v) {
  return wave_reduce(v, [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

}  // namespace ix
