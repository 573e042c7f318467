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
// position pos0 + 64 j + l (ascending in (j, l)); valid[j] marks the lanes
// whose value j exists.  A kLocalBins-bin histogram over the wave's [min, max]
// (in hist, kLocalBins words of LDS private to the wave) gives the bin holding
// the (cap+1)-th best; the values in higher bins are kept.  They go to
// dst[0..kept) in position order as (order key, position).  Returns the
// piece's record (kept, largest dropped order key or 0, smallest and largest
// kept order key or ~0 / 0), uniform over the wave.
template <int NV>
__device__ __forceinline__ uint4 wave_keep_top(const float (&v)[NV], const uint64_t (&valid)[NV], int pos0,
                                               int cap, uint32_t* hist, uint2* __restrict__ dst) {
  const int l = lane_id();
  int n = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) n += __popcll(valid[j]);
  int vb = -1;                             // keep values in bins above vb
  float lo = 0.0f, inv = 0.0f;
  if (n > cap) {
    float hi = -INFINITY;
    lo = INFINITY;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((valid[j] >> l) & 1u) {
        lo = fminf(lo, v[j]);
        hi = fmaxf(hi, v[j]);
      }
    lo = wave_min(lo);
    hi = wave_max(hi);
    inv = (float)kLocalBins / (hi - lo);
    if (!(hi > lo) || !(inv > 0.0f) || !(inv < INFINITY)) inv = 0.0f;   // one bin: keep nothing
    *reinterpret_cast<u32x4*>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((valid[j] >> l) & 1u) atomicAdd(&hist[min(kLocalBins - 1, max(0, (int)((v[j] - lo) * inv)))], 1u);
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
  }
  int out = 0;
  uint32_t dropped = 0u, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const bool in = (valid[j] >> l) & 1u;
    const bool keep = in && min(kLocalBins - 1, max(0, (int)((v[j] - lo) * inv))) > vb;
    const uint64_t km = __ballot(keep);
    const uint32_t key = order_key(v[j]);
    if (keep) {
      dst[out + wave_prefix(km)] = make_uint2(key, (uint32_t)(pos0 + 64 * j + l));
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    } else if (in) {
      dropped = max(dropped, key);
    }
    out += __popcll(km);
  }
  return make_uint4((uint32_t)out, wave_max(dropped), wave_min(kmin), wave_max(kmax));
}

}  // namespace ix
