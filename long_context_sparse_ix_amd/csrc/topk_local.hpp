// Wave-local first stage of the few-long-rows top-k (gfx950).
//
// A long score row is cut into pieces of NV x 64 consecutive positions, one
// wave per piece.  A row of P pieces gives each piece kLocalCap / P slots of
// the row's candidate list: the wave keeps at most that many of its scores,
// the ones in the value bins above the bin holding its (cap+1)-th best, and
// records the largest order key it dropped.  The merge pass then selects the
// row's k best among the kept entries, which is exact whenever that k-th best
// is above every dropped key (see topk_rows.hip).  Everything here is one
// wave: a histogram in the wave's own LDS words, ballots and register-level
// lane exchanges, no barriers, so the stage can also run as the epilogue of
// the score kernel.
#pragma once

#include "device_common.hpp"

namespace ix {

constexpr int kLocalCap = 8192;       // candidate slots per row (all pieces together)
constexpr int kLocalMaxPieces = 512;  // at least 16 slots per piece
constexpr int kLocalBins = 256;       // value bins of a wave's histogram (4 per lane)

// Keeps at most cap of this wave's valid values.  Lane l's value j sits at
// position pos0 + 64 j + l (ascending in (j, l)) and is valid when
// 64 j + l < rem (the wave's valid positions are a prefix of length rem, which
// may be <= 0 or beyond NV * 64).  A kLocalBins-bin histogram over the wave's
// [min, max] (in hist, kLocalBins words of LDS private to the wave) gives the
// bin holding the (cap+1)-th best; the values in higher bins are kept (all of
// them when there are at most cap).  They go to dst[0..kept) in position
// order as (order key, position).  Returns the piece's record (kept, largest
// dropped order key or 0, smallest and largest kept order key or ~0 / 0),
// uniform over the wave.  Each value's bin is computed once and reused.
template <int NV>
__device__ __forceinline__ uint4 wave_keep_top(const float (&v)[NV], int rem, int pos0, int cap, uint32_t* hist,
                                               uint2* __restrict__ dst) {
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
