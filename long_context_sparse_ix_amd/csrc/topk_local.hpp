// Wave-local first stage of the few-long-rows top-k (gfx950).
//
// A long score row is cut into pieces of NV x 64 consecutive positions, one
// wave per piece.  A row of P pieces gives each piece kLocalCap / P slots of
// the row's candidate list: the wave keeps at most that many of its scores,
// the ones in the value bins above the bin holding its (cap+1)-th best, and
// records a bound D at or above every order key it dropped.  The merge pass
// then selects the row's k best among the kept entries, which is exact
// whenever that k-th best is above every piece's D (see topk_rows.hip).  Everything here is one
// wave: a histogram in the wave's own LDS words, ballots and register-level
// lane exchanges, no barriers, so the stage can also run as the epilogue of
// the score kernel.
#pragma once

#include "device_common.hpp"

namespace ix {

constexpr int kLocalCap = 8192;       // candidate slots per row (all pieces together)
constexpr int kLocalMaxPieces = 512;  // at least 16 slots per piece
constexpr int kLocalBins = 256;       // value bins of a wave's histogram (4 per lane)

// wave_keep_top for a wave whose NV * 64 values are all valid, with fewer
// instructions per value:
//  - the bins come from one saturating float -> u8 conversion (rounded, so
//    monotone in the value; the keep test and the histogram use the same
//    bin);
//  - the kept entries are stored through a buffer resource over the piece's
//    cap slots (32-bit offsets);
//  - D is one below the smallest kept key: a kept value's bin is above vb and
//    a dropped one's at or below it, so with monotone bins every kept value
//    is above every dropped one (D is the largest dropped key itself when
//    nothing is kept, 0 when nothing is dropped);
//  - the largest kept key is the wave maximum's (its bin is the highest).
template <int NV>
__device__ __forceinline__ uint4 wave_keep_top_full(const float (&v)[NV], int pos0, int cap, uint32_t* hist,
                                                    uint2* __restrict__ dst) {
  const int l = lane_id();
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) {
    lo = fminf(lo, v[j]);
    hi = fmaxf(hi, v[j]);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  uint32_t bn[NV];
  int vb = -1;
  if (NV * kWave > cap) {
    float inv = (float)kLocalBins / (hi - lo);
    if (!(hi > lo) || !(inv > 0.0f) || !(inv < INFINITY)) inv = 0.0f;   // one bin: keep nothing
    *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      bn[j] = __builtin_amdgcn_cvt_pk_u8_f32((v[j] - lo) * inv, 0, 0u);
      atomicAdd(&hist[bn[j]], 1u);
    }
    wave_lds_sync();
    const int kk = cap + 1;
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const int tot = (int)(h.x + h.y + h.z + h.w);
    const int a3 = (int)wave_suffix_sum((uint32_t)tot) - tot;
    const int a2 = a3 + (int)h.w, a1 = a2 + (int)h.z, a0 = a1 + (int)h.y;
    // one lane holds the (cap+1)-th best (there are NV * 64 > cap values)
    const uint64_t bm = __ballot(a3 < kk && kk <= a3 + tot);
    const int bin = 4 * l + 3 - (int)(kk > a2) - (int)(kk > a1) - (int)(kk > a0);
    vb = __builtin_amdgcn_readlane(bin, (int)__builtin_ctzll(bm));
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) bn[j] = 0u;
  }
  int out = 0;
  uint32_t kmin = 0xFFFFFFFFu;
  const uint32_t pl = (uint32_t)(pos0 + l);
  // the piece's cap slots, addressed by 32-bit offsets
  const uint64_t da = reinterpret_cast<uint64_t>(dst);   // uniform over the wave
  const uint64_t du = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)da) |
                      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(da >> 32)) << 32);
  const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(du), (short)0, __builtin_amdgcn_readfirstlane(cap * 8), 0x00020000);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool keep = (int)bn[j] > vb;
    const uint64_t km = __ballot(keep);
    if (keep) {
      // order key of v + 0 (-0 and +0 share the key of +0)
      const uint32_t u = __float_as_uint(v[j] + 0.0f);
      const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
      const u32x2v e = {key, pl + (uint32_t)(kWave * j)};
      __builtin_amdgcn_raw_buffer_store_b64(e, dr, (out + wave_prefix(km)) * 8, 0, 0);   // at most cap are kept
      kmin = min(kmin, key);
    }
    out += __popcll(km);
  }
  kmin = wave_min(kmin);
  const uint32_t dropped = out == NV * kWave ? 0u : out == 0 ? order_key(hi) : kmin - 1u;
  return make_uint4((uint32_t)out, dropped, kmin, out > 0 ? order_key(hi) : 0u);
}

// Keeps at most cap of this wave's valid values.  Lane l's value j sits at
// position pos0 + 64 j + l (ascending in (j, l)) and is valid when
// 64 j + l < rem (the wave's valid positions are a prefix of length rem, which
// may be <= 0 or beyond NV * 64).  A kLocalBins-bin histogram over the wave's
// [min, max] (in hist, kLocalBins words of LDS private to the wave) gives the
// bin holding the (cap+1)-th best; the values in higher bins are kept (all of
// them when there are at most cap).  They go to dst[0..kept) in position
// order as (order key, position).  Returns the piece's record (kept, D,
// smallest and largest kept order key or ~0 / 0), uniform over the wave; on
// a partly valid wave D is the largest dropped key (0 when none is dropped).
// Each value's bin is computed once and reused.
template <int NV>
__device__ __forceinline__ uint4 wave_keep_top(const float (&v)[NV], int rem, int pos0, int cap, uint32_t* hist,
                                               uint2* __restrict__ dst) {
  if (rem >= NV * kWave) return wave_keep_top_full<NV>(v, pos0, cap, hist, dst);
  const int l = lane_id();
  const int lim = rem - l;                 // value j of this lane is valid when 64 j < lim
  const int n = rem <= 0 ? 0 : (rem < NV * kWave ? rem : NV * kWave);
  int bn[NV];                              // value bin, or -1 for an invalid value
  int vb = -1;                             // keep values in bins above vb
  if (n > cap) {
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (kWave * j < lim) {
        lo = fminf(lo, v[j]);
        hi = fmaxf(hi, v[j]);
      }
    lo = wave_min(lo);
    hi = wave_max(hi);
    float inv = (float)kLocalBins / (hi - lo);
    if (!(hi > lo) || !(inv > 0.0f) || !(inv < INFINITY)) inv = 0.0f;   // one bin: keep nothing
    *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      bn[j] = kWave * j < lim ? min(kLocalBins - 1, max(0, (int)((v[j] - lo) * inv))) : -1;
      if (bn[j] >= 0) atomicAdd(&hist[bn[j]], 1u);
    }
    wave_lds_sync();
    // bin holding the (cap+1)-th best: lane l owns bins 4l .. 4l+3
    const int kk = cap + 1;
    const u32x4 h = *reinterpret_cast<const u32x4*>(hist + 4 * l);
    const int tot = (int)(h.x + h.y + h.z + h.w);
    const int a3 = (int)wave_suffix_sum((uint32_t)tot) - tot;     // values in higher lanes' bins
    const int a2 = a3 + (int)h.w, a1 = a2 + (int)h.z, a0 = a1 + (int)h.y;
    int bin = -1;
    if (a3 < kk && kk <= a2) bin = 4 * l + 3;
    else if (a2 < kk && kk <= a1) bin = 4 * l + 2;
    else if (a1 < kk && kk <= a0) bin = 4 * l + 1;
    else if (a0 < kk && kk <= a0 + (int)h.x) bin = 4 * l;
    const uint64_t bm = __ballot(bin >= 0);
    vb = __shfl(bin, __ffsll((unsigned long long)bm) - 1);
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) bn[j] = kWave * j < lim ? 0 : -1;
  }
  int out = 0;
  uint32_t dropped = 0u, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool keep = bn[j] > vb;
    const uint64_t km = __ballot(keep);
    const uint32_t key = order_key(v[j]);
    if (keep) {
      const int o = out + wave_prefix(km);
      if (o < cap) dst[o] = make_uint2(key, (uint32_t)(pos0 + 64 * j + l));   // at most cap are kept
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    } else if (bn[j] >= 0) {
      dropped = max(dropped, key);
    }
    out += __popcll(km);
  }
  return make_uint4((uint32_t)out, wave_max(dropped), wave_min(kmin), wave_max(kmax));
}

}  // namespace ix
