// Per-row top-k over materialised fp32 score rows.
//
// Selection rule ("IndexShare", LLM Architecture Gallery, section "How
// IndexShare Works": a full layer runs the top-k itself and keeps the chosen
// positions for the shared layers): keep the min(k, p+1) best positions of row p under
// (score desc, position asc); emit them in ascending position order, then -1.
//
// Few long rows (decode: 32 rows of ~200K scores) cannot fill the chip with one
// workgroup per row, so the work of a row is spread over many waves.  Rows of
// up to 512 pieces of 1024 positions (524,288 scores) take two passes:
//   K  keep:   one wave per piece (the score kernel's waves keep their own 640
//              scores the same way, as their epilogue) keeps at most
//              cap = 8192 / P of its scores, P the row's piece count: a
//              256-bin value histogram in the wave's own LDS words gives the
//              bin holding its (cap+1)-th best, and every score in a higher
//              bin is kept, in position order, at slots [c*cap, ...) of the
//              row's candidate list.  The piece records how many it kept, a
//              bound D at or above every key it dropped, and its kept key
//              range (topk_local.hpp);
//   M  merge:  per row, one workgroup holds the whole candidate list in
//              registers and selects the k best of the entries above the
//              largest D; if at least k lie above it, no dropped score can
//              rank among the k best, and a stable emission writes the row.
//              Otherwise (a ramp that puts the winners in one piece, a flat
//              row) the row is finished by a single-workgroup exact select
//              over the whole row.
// Random rows keep about 4x what each piece contributes to the top k (k <=
// 2048 of 8192 slots), so the fallback is rare.  Longer rows run five passes
// over chunks of 8192 scores, each with its own workgroup:
//   R  range:   min / max of every chunk;
//   H  hist:    a 1024-bin value-domain histogram of every chunk over the
//               row's [min, max] (bins are monotone in the score);
//   S  select:  per row, the bin vb holding the k-th best, the number m of
//               scores in bins >= vb and, per chunk, where its share of those
//               m starts in the row's candidate list;
//   C  collect: every chunk writes its scores in bins >= vb, in position order,
//               as (order key, position) into the candidate list;
//   F  finish:  per row, an exact radix select over the m candidates in LDS
//               gives the k-th key v and how many ties at v are kept, then a
//               stable pass over the list (already in position order) emits.
// A row whose m exceeds the candidate capacity (a flat or adversarial score
// distribution) is finished instead by a single-workgroup exact select over
// the whole row.  Many-row calls use that single-workgroup select directly: one
// workgroup per row already fills the chip and needs no workspace.
#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_local.hpp"

namespace ix {

namespace {

constexpr int kCT = 512;                 // threads of the chunk passes
constexpr int kPT = 16;                  // scores per thread in a chunk pass
constexpr int kChunk = kCT * kPT;        // 8192 scores per chunk
constexpr int kVB = 1024;                // value bins of a chunk histogram
constexpr int kST = 256;                 // threads of the select pass (4 bins each)
constexpr int kFT = 1024;                // threads of the finish / single-row select
constexpr int kCap = kLocalCap;          // candidate capacity per row
constexpr int kMultiRowLimit = 1024;     // rows below this use the chunked select

constexpr int kSingleBins = 2048;        // value bins of the single-workgroup select

// Row state handed from S to C and F.
struct RowSel {
  float lo, inv;   // value binning of the row
  int vb;          // bin holding the k-th best
  int m;           // scores in bins >= vb; kFallback / kTrivial as below
  int above;       // scores in bins > vb
  int pad[3];
};
constexpr int kFallback = -1;            // too many candidates: whole-row select
constexpr int kTrivial = -2;             // p + 1 <= k: keep every position

// Candidates of row `row` (= b * n_q + t): positions 0 .. start_b + t.
__device__ __forceinline__ int row_len(int row, int n_q, int64_t q_start, const int64_t* seq) {
  return (int)(seq_start(seq, row / n_q, q_start) + row % n_q + 1);
}

__device__ __forceinline__ int vbin(float s, float lo, float inv, int nbins) {
  return min(nbins - 1, max(0, (int)((s - lo) * inv)));
}

// Bin scale over [lo, hi]; 0 (every score in bin 0) when the range cannot be
// split.
__device__ __forceinline__ float bin_scale(float lo, float hi, int nbins) {
  float inv = nbins / (hi - lo);
  if (!(hi > lo) || !(inv > 0.0f) || !(inv < INFINITY)) inv = 0.0f;
  return inv;
}

// ---- block-wide helpers (NT threads, one LDS slot per wave) ----

template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* red, Op op) {
  v = wave_reduce(v, op);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  T r = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = op(r, red[w]);
  __syncthreads();
  return r;
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* red, int* total) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (l >= d) x += y;
  }
  if (l == kWave - 1) red[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    const int s = red[i];
    before += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

struct MinOp { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct UMinOp { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct UMaxOp { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

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

// The kk-th largest of the order keys key(i), i in [0, n), among those with
// pred(i), by 8-bit radix passes over key - kmin (kmin/kmax: the range of the
// keys that pass pred).  Returns v; *need = kk - #{key > v}, the ties at v
// that are kept.  hist holds >= 256 words of LDS.
template <int NT, typename KeyF, typename PredF>
__device__ uint32_t radix_kth(int n, int kk, uint32_t kmin, uint32_t kmax, KeyF key, PredF pred,
                              uint32_t* hist, int* sel_bin, int* sel_above, int* need) {
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0u ? 0 : 32 - __clz((int)range);
  uint32_t prefix = 0u, pmask = 0u;
  for (int shift = ((nbits + 7) & ~7) - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      if (!pred(i)) continue;
      const uint32_t rel = key(i) - kmin;
      if ((rel & pmask) == prefix) atomicAdd(&hist[(rel >> shift) & 255u], 1u);
    }
    __syncthreads();
    pick_from_top(hist, 256, kk, sel_bin, sel_above);
    kk -= *sel_above;
    prefix |= (uint32_t)*sel_bin << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  *need = kk;
  return kmin + prefix;
}

// The kk-th largest order key among entries i in [0, n) with pred(i), whose
// keys lie in [kmin, kmax]: a kSingleBins value histogram over that range
// gives the bin holding it (the bins spread a tail of scores thinly, where the
// top 8 bits of the keys would pile most of them into a few bins and
// serialise the LDS atomics), then the exact radix select runs over that
// bin's entries only.  hist holds >= kSingleBins words of LDS.
template <int NT, typename KeyF, typename PredF>
__device__ uint32_t select_binned(int n, int kk, uint32_t kmin, uint32_t kmax, KeyF key, PredF pred,
                                  uint32_t* hist, uint32_t* redu, int* sel_bin, int* sel_above, int* need) {
  const float lo = key_value(kmin);
  const float inv = bin_scale(lo, key_value(kmax), kSingleBins);
  for (int i = threadIdx.x; i < kSingleBins; i += NT) hist[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT)
    if (pred(i)) atomicAdd(&hist[vbin(key_value(key(i)), lo, inv, kSingleBins)], 1u);
  __syncthreads();
  pick_from_top(hist, kSingleBins, kk, sel_bin, sel_above);
  const int vb = *sel_bin;
  const int kb = kk - *sel_above;
  const auto in_vb = [&](int i) { return pred(i) && vbin(key_value(key(i)), lo, inv, kSingleBins) == vb; };
  uint32_t bmin = 0xFFFFFFFFu, bmax = 0u;
  for (int i = threadIdx.x; i < n; i += NT)
    if (in_vb(i)) {
      bmin = min(bmin, key(i));
      bmax = max(bmax, key(i));
    }
  bmin = block_reduce<NT>(bmin, redu, UMinOp{});
  bmax = block_reduce<NT>(bmax, redu, UMaxOp{});
  return radix_kth<NT>(n, kb, bmin, bmax, key, in_vb, hist, sel_bin, sel_above, need);
}

// ---- single-workgroup select of one whole row (kFT threads) ----
//   1. min / max of the row;  2. a 2048-bin value histogram gives the bin
//   holding the k-th best;  3. exact radix select on the order keys of that
//   bin's entries;  4. stable emission in position order.
__device__ void select_row_single(const float* __restrict__ src, int n, int k, int32_t* __restrict__ dst) {
  __shared__ uint32_t hist[kSingleBins];
  __shared__ float redf[kFT / kWave];
  __shared__ uint32_t redu[kFT / kWave];
  __shared__ int sel_bin, sel_above;
  __shared__ int wave_keep[kFT / kWave], wave_eq[kFT / kWave];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;

  float a = INFINITY, b = -INFINITY;
  for (int i = tid; i < n; i += kFT) {
    const float s = src[i];
    a = fminf(a, s);
    b = fmaxf(b, s);
  }
  const float lo = block_reduce<kFT>(a, redf, MinOp{});
  const float hi = block_reduce<kFT>(b, redf, MaxOp{});
  const float inv = bin_scale(lo, hi, kSingleBins);

  for (int i = tid; i < kSingleBins; i += kFT) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kFT) atomicAdd(&hist[vbin(src[i], lo, inv, kSingleBins)], 1u);
  __syncthreads();
  pick_from_top(hist, kSingleBins, k, &sel_bin, &sel_above);
  const int vb = sel_bin;
  const int kk = k - sel_above;
  __syncthreads();

  uint32_t a_min = 0xFFFFFFFFu, a_max = 0u;
  for (int i = tid; i < n; i += kFT) {
    const float s = src[i];
    if (vbin(s, lo, inv, kSingleBins) == vb) {
      const uint32_t key = order_key(s);
      a_min = min(a_min, key);
      a_max = max(a_max, key);
    }
  }
  const uint32_t kmin = block_reduce<kFT>(a_min, redu, UMinOp{});
  const uint32_t kmax = block_reduce<kFT>(a_max, redu, UMaxOp{});
  int need = 0;
  const uint32_t v = radix_kth<kFT>(
      n, kk, kmin, kmax, [&](int i) { return order_key(src[i]); },
      [&](int i) { return vbin(src[i], lo, inv, kSingleBins) == vb; }, hist, &sel_bin, &sel_above, &need);

  int out_base = 0, eq_base = 0;
  for (int base = 0; base < n; base += kFT) {
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
    const int o = keep_before + wave_prefix(km);
    if (keep && o < k) dst[o] = i;
    int kt = 0, et = 0;
    for (int w = 0; w < kFT / kWave; ++w) { kt += wave_keep[w]; et += wave_eq[w]; }
    out_base += kt;
    eq_base += et;
    __syncthreads();
  }
}

__device__ void write_trivial(int32_t* dst, int n, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) dst[i] = i < n ? i : -1;
}

__global__ __launch_bounds__(kFT) void topk_rows_single_kernel(const float* __restrict__ scores, int64_t ld,
                                                               int32_t* __restrict__ idx, int n_q,
                                                               int64_t q_start, const int64_t* seq,
                                                               int k) {
  const int row = blockIdx.x;
  const int n = row_len(row, n_q, q_start, seq);
  int32_t* dst = idx + (int64_t)row * k;
  if (n <= k) {
    write_trivial(dst, n, k);
    return;
  }
  select_row_single(scores + (int64_t)row * ld, n, k, dst);
}

// ---- chunked passes ----

struct ChunkArgs {
  const float* scores;
  int64_t ld;
  int n_q;
  int64_t q_start;
  const int64_t* seq;   // nullable: per-sequence start of row 0
  int k;
  int G;           // chunks per row (of the longest row)
  int vec;         // rows are 16-byte aligned: load float4
  const float2* rng;  // range partials: [rows][rng_stride], one per rng_span scores
  int rng_span, rng_stride;
  float2* rng_own;    // [rows][G], written by the range pass when no partials are given
  uint4* local;       // [rows][local_stride] per piece: kept count, largest dropped order key,
                      // smallest and largest kept order key
  int local_stride, local_span;   // pieces of local_span positions
  uint32_t* hist;  // [rows][G][kVB]
  int32_t* off;    // [rows][G]
  RowSel* sel;     // [rows]
  uint2* cand;     // [rows][kCap]
};

// This thread's kPT scores, positions i0 .. i0 + kPT - 1 (entries at or
// beyond n are not read and must be masked by the caller).
__device__ __forceinline__ void load_run(const float* __restrict__ row, int i0, int n, bool vec,
                                         float (&v)[kPT]) {
  if (vec && i0 + kPT <= n) {
#pragma unroll
    for (int j = 0; j < kPT / 4; ++j) {
      const float4 x = *reinterpret_cast<const float4*>(row + i0 + 4 * j);
      v[4 * j] = x.x;
      v[4 * j + 1] = x.y;
      v[4 * j + 2] = x.z;
      v[4 * j + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPT; ++j) v[j] = i0 + j < n ? row[i0 + j] : 0.0f;
  }
}

// lo / inv of a row from its chunks' ranges (all threads of the block).
template <int NT>
__device__ __forceinline__ void row_binning(const float2* rng, int G, float* red, float& lo, float& inv) {
  float a = INFINITY, b = -INFINITY;
  for (int g = threadIdx.x; g < G; g += NT) {
    const float2 r = rng[g];
    a = fminf(a, r.x);
    b = fmaxf(b, r.y);
  }
  lo = block_reduce<NT>(a, red, MinOp{});
  const float hi = block_reduce<NT>(b, red, MaxOp{});
  inv = bin_scale(lo, hi, kVB);
}

__global__ __launch_bounds__(kCT) void tk_range_kernel(ChunkArgs a) {
  __shared__ float red[kCT / kWave];
  const int row = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  const int base = g * kChunk;
  if (n <= a.k || base >= n) return;
  const int i0 = base + threadIdx.x * kPT;
  float v[kPT];
  load_run(a.scores + (int64_t)row * a.ld, i0, n, a.vec, v);
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPT; ++j)
    if (i0 + j < n) {
      mn = fminf(mn, v[j]);
      mx = fmaxf(mx, v[j]);
    }
  mn = block_reduce<kCT>(mn, red, MinOp{});
  mx = block_reduce<kCT>(mx, red, MaxOp{});
  if (threadIdx.x == 0) a.rng_own[(int64_t)row * a.G + g] = make_float2(mn, mx);
}

__global__ __launch_bounds__(kCT) void tk_hist_kernel(ChunkArgs a) {
  __shared__ uint32_t h[kVB];
  __shared__ float red[kCT / kWave];
  const int row = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  const int base = g * kChunk;
  if (n <= a.k || base >= n) return;
  const int i0 = base + threadIdx.x * kPT;
  float v[kPT];
  load_run(a.scores + (int64_t)row * a.ld, i0, n, a.vec, v);
  for (int i = threadIdx.x; i < kVB; i += kCT) h[i] = 0u;
  float lo, inv;
  row_binning<kCT>(a.rng + (int64_t)row * a.rng_stride, (n + a.rng_span - 1) / a.rng_span, red, lo, inv);
#pragma unroll
  for (int j = 0; j < kPT; ++j)
    if (i0 + j < n) atomicAdd(&h[vbin(v[j], lo, inv, kVB)], 1u);
  __syncthreads();
  uint32_t* dst = a.hist + ((int64_t)row * a.G + g) * kVB;
  for (int i = threadIdx.x; i < kVB; i += kCT) dst[i] = h[i];
}

__global__ __launch_bounds__(kST) void tk_select_kernel(ChunkArgs a) {
  __shared__ float red[kST / kWave];
  __shared__ int redi[kST / kWave];
  __shared__ int sh_vb, sh_above, sh_h;
  __shared__ int cnt[kST];                       // per-chunk counts, kST at a time
  const int row = blockIdx.x, tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  if (n <= a.k) {
    if (tid == 0) a.sel[row] = RowSel{0.0f, 0.0f, 0, kTrivial, 0, {}};
    return;
  }
  const int Gr = (n + kChunk - 1) / kChunk;
  float lo, inv;
  row_binning<kST>(a.rng + (int64_t)row * a.rng_stride, (n + a.rng_span - 1) / a.rng_span, red, lo, inv);

  // row histogram: bins 4*tid .. 4*tid + 3
  const uint32_t* hb = a.hist + (int64_t)row * a.G * kVB;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int g0 = 0; g0 < Gr; g0 += 8) {          // 8 chunk loads in flight
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = g0 + j < Gr ? *reinterpret_cast<const u32x4*>(hb + (int64_t)(g0 + j) * kVB + 4 * tid)
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += x[j];
  }
  const int tot = (int)(acc.x + acc.y + acc.z + acc.w);
  // entries in bins above this thread's: total minus inclusive prefix
  int all;
  const int before = block_excl_scan<kST>(tot, redi, &all);
  int ab = all - before - tot;
  const int hs[4] = {(int)acc.x, (int)acc.y, (int)acc.z, (int)acc.w};
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (ab < a.k && a.k <= ab + hs[j]) {
      sh_vb = 4 * tid + j;
      sh_above = ab;
      sh_h = hs[j];
    }
    ab += hs[j];
  }
  __syncthreads();
  const int vb = sh_vb;
  const int m = sh_above + sh_h;
  if (m > kCap) {
    if (tid == 0) a.sel[row] = RowSel{lo, inv, vb, kFallback, 0, {}};
    return;
  }
  // per-chunk counts of bins >= vb (one wave per chunk, 16 bins per lane),
  // then their exclusive prefix in chunk order, kST chunks at a time
  int carry = 0;
  for (int g0 = 0; g0 < Gr; g0 += kST) {
    const int gn = min(kST, Gr - g0);
    for (int gi0 = wave; gi0 < gn; gi0 += 2 * (kST / kWave)) {   // two chunks per wave at once
      u32x4 x[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int gi = gi0 + u * (kST / kWave);
        const uint32_t* hc = hb + (int64_t)(g0 + (gi < gn ? gi : 0)) * kVB + 16 * l;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = *reinterpret_cast<const u32x4*>(hc + 4 * j);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int gi = gi0 + u * (kST / kWave);
        int c = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b0 = 16 * l + 4 * j;
          c += (b0 >= vb ? (int)x[u][j].x : 0) + (b0 + 1 >= vb ? (int)x[u][j].y : 0) +
               (b0 + 2 >= vb ? (int)x[u][j].z : 0) + (b0 + 3 >= vb ? (int)x[u][j].w : 0);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
        if (l == 0 && gi < gn) cnt[gi] = c;
      }
    }
    __syncthreads();
    const int c = tid < gn ? cnt[tid] : 0;
    int chunk_tot;
    const int ex = block_excl_scan<kST>(c, redi, &chunk_tot);
    if (tid < gn) a.off[(int64_t)row * a.G + g0 + tid] = carry + ex;
    carry += chunk_tot;
  }
  if (tid == 0) a.sel[row] = RowSel{lo, inv, vb, m, sh_above, {}};
}

__global__ __launch_bounds__(kCT) void tk_collect_kernel(ChunkArgs a) {
  __shared__ int redi[kCT / kWave];
  const int row = blockIdx.x / a.G, g = blockIdx.x % a.G;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  const int base = g * kChunk;
  if (n <= a.k || base >= n) return;
  const RowSel rs = a.sel[row];
  if (rs.m < 0) return;
  const int i0 = base + threadIdx.x * kPT;
  float v[kPT];
  load_run(a.scores + (int64_t)row * a.ld, i0, n, a.vec, v);
  uint32_t take = 0u;
#pragma unroll
  for (int j = 0; j < kPT; ++j)
    if (i0 + j < n && vbin(v[j], rs.lo, rs.inv, kVB) >= rs.vb) take |= 1u << j;
  int total;
  const int ex = block_excl_scan<kCT>(__popc(take), redi, &total);
  uint2* dst = a.cand + (int64_t)row * kCap;
  int o = a.off[(int64_t)row * a.G + g] + ex;
#pragma unroll
  for (int j = 0; j < kPT; ++j)
    if ((take & (1u << j)) && o < rs.m) dst[o++] = make_uint2(order_key(v[j]), (uint32_t)(i0 + j));
}

// Candidate lists in LDS are stored with one pad word after every 8 entries:
// the stable emission gives each thread a run of up to 8 consecutive entries,
// and with the pad the 64 lanes of a wave read 64 different banks instead of
// 8 lanes per bank.
constexpr int kCapPadded = kCap + kCap / 8;
__device__ __forceinline__ int lds_at(int i) { return i + (i >> 3); }

// Exclusive prefix sum over the kFT threads in thread order, one barrier
// (wtot: kFT / kWave words of LDS used by this call only).
__device__ __forceinline__ uint32_t block_excl_scan1(uint32_t v, uint32_t* wtot) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (l == kWave - 1) wtot[w] = x;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += wtot[i];
  return before + x - v;
}

// Stable emission of a position-ordered candidate list (keys ck, positions
// cp, m <= 8192 entries in LDS at lds_at(i)): every entry with key > v and the
// first `need` with key == v, in list order.  Thread t owns entries [t*P,
// t*P + P).  One scan of the packed per-thread counts (key > v in the low 16
// bits, key == v in the high 16) places every thread's output: the ties kept
// before it are min(ties before it, need).
__device__ __forceinline__ void emit_stable(const uint32_t* ck, const int* cp, int m, uint32_t v, int need,
                                            int k, int32_t* __restrict__ dst, uint32_t* wtot) {
  const int tid = threadIdx.x;
  const int P = (m + kFT - 1) / kFT;
  const int e0 = min(m, tid * P), e1 = min(m, e0 + P);
  uint32_t gt = 0, eq = 0;
  for (int i = e0; i < e1; ++i) {
    const uint32_t key = ck[lds_at(i)];
    gt += key > v;
    eq += key == v;
  }
  const uint32_t ex = block_excl_scan1(gt | (eq << 16), wtot);
  int eq_rank = (int)(ex >> 16);
  int out = (int)(ex & 0xFFFFu) + min(eq_rank, need);
  for (int i = e0; i < e1 && out < k; ++i) {
    const uint32_t key = ck[lds_at(i)];
    if (key > v || (key == v && eq_rank++ < need)) dst[out++] = cp[lds_at(i)];
  }
}

__global__ __launch_bounds__(kFT) void tk_finish_kernel(ChunkArgs a, int32_t* __restrict__ idx) {
  __shared__ uint32_t ck[kCapPadded];
  __shared__ int cp[kCapPadded];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t redu[kFT / kWave];
  __shared__ uint32_t wtot[kFT / kWave];
  __shared__ int sel_bin, sel_above;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  int32_t* dst = idx + (int64_t)row * a.k;
  const RowSel rs = a.sel[row];
  if (rs.m == kTrivial) {
    write_trivial(dst, n, a.k);
    return;
  }
  if (rs.m == kFallback) {
    select_row_single(a.scores + (int64_t)row * a.ld, n, a.k, dst);
    return;
  }
  const int m = rs.m;
  const uint2* src = a.cand + (int64_t)row * kCap;
  // every candidate in a bin above vb is kept; the k-th best is the
  // (k - above)-th among bin vb's, whose key range is narrow
  const auto in_vb = [&](uint32_t key) { return vbin(key_value(key), rs.lo, rs.inv, kVB) == rs.vb; };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int i = tid; i < m; i += kFT) {
    const uint2 e = src[i];
    ck[lds_at(i)] = e.x;
    cp[lds_at(i)] = (int)e.y;
    if (in_vb(e.x)) {
      kmin = min(kmin, e.x);
      kmax = max(kmax, e.x);
    }
  }
  kmin = block_reduce<kFT>(kmin, redu, UMinOp{});
  kmax = block_reduce<kFT>(kmax, redu, UMaxOp{});   // its barriers publish ck / cp
  int need = 0;
  const uint32_t v = radix_kth<kFT>(
      m, a.k - rs.above, kmin, kmax, [&](int i) { return ck[lds_at(i)]; }, [&](int i) { return in_vb(ck[lds_at(i)]); }, hist,
      &sel_bin, &sel_above, &need);

  emit_stable(ck, cp, m, v, need, a.k, dst, wtot);
}

// ---- wave-local keep + merge (rows of at most kLocalMaxPieces pieces) ----

constexpr int kLocalNV = 16;                    // scores per lane of a standalone piece
constexpr int kLocalSpan = kLocalNV * kWave;    // 1024 positions per piece

__global__ __launch_bounds__(256) void tk_wave_local_kernel(ChunkArgs a) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int row = blockIdx.y, piece = blockIdx.x * 4 + wave;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  if (n <= a.k) return;
  const int P = (n + kLocalSpan - 1) / kLocalSpan;
  if (piece >= P) return;
  const int pos0 = piece * kLocalSpan;
  const float* src = a.scores + (int64_t)row * a.ld;
  float v[kLocalNV];
  if (pos0 + kLocalSpan <= n) {
#pragma unroll
    for (int j = 0; j < kLocalNV; ++j) v[j] = src[pos0 + kWave * j + l];
  } else {
#pragma unroll
    for (int j = 0; j < kLocalNV; ++j) v[j] = src[min(pos0 + kWave * j + l, n - 1)];
  }
  const int cap = kLocalCap / P;
  __shared__ uint32_t hist[4][kLocalBins];
  const uint4 r = wave_keep_top<kLocalNV>(v, n - pos0, pos0, cap, hist[wave],
                                          a.cand + (int64_t)row * kLocalCap + (int64_t)piece * cap);
  if (l == 0) a.local[(int64_t)row * a.local_stride + piece] = r;
}

// Per row: the pieces' kept entries (piece c at slots [c*cap, c*cap + kept_c)
// of the candidate list, in position order).  D, the largest of the pieces'
// bounds, is at or above every dropped key; if at least k entries lie above
// D, the row's k-th best is among them and every dropped entry ranks below
// it, so the k-th best of the entries above D and a stable emission give the
// row's top k.  Otherwise the whole-row select runs.
// Thread t holds the 8 contiguous slots [8t, 8t + 8) in registers, so the
// valid entries' list order is thread order and nothing is copied to LDS:
//   A  every thread loads its slots and one piece's record at once; per-wave
//      sums / extremes of the records and one barrier give the kept count m,
//      D and the kept key range;
//   B  valid slots above D go into a kMergeBins value histogram over
//      (D, largest kept];
//   C  one wave finds the bin holding the k-th best;
//   D  that bin's keys form a short list (all above D, so every tie of the
//      k-th key is in it);
//   E  one wave ranks the short list (one key per lane) for the k-th key v and
//      the number of its ties to keep; a longer list runs the radix select;
//   F  stable emission: one scan of per-thread counts places each thread's
//      kept positions.
constexpr int kShort = 1024;            // short-list capacity (else the whole-row select runs)
constexpr int kMergeBins = 1024;
constexpr int kMergeSlots = kLocalCap / kFT;   // contiguous candidate slots per thread
static_assert(kMergeSlots == 8, "two 16-byte loads of two slots, twice");

__global__ __launch_bounds__(kFT) void tk_merge_kernel(ChunkArgs a, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kMergeBins];
  __shared__ uint32_t sk[kShort];
  __shared__ int kept[kLocalMaxPieces];
  __shared__ uint4 wpart[kFT / kWave];
  __shared__ int wabove[kFT / kWave];
  __shared__ uint32_t wtot[kFT / kWave];
  __shared__ uint32_t redu[kFT / kWave];
  __shared__ int sel_bin, sel_above, sh_short, sh_need;
  __shared__ uint32_t sh_v;
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int n = row_len(row, a.n_q, a.q_start, a.seq);
  int32_t* dst = idx + (int64_t)row * a.k;
  if (n <= a.k) {
    write_trivial(dst, n, a.k);
    return;
  }
  const int P = (n + a.local_span - 1) / a.local_span;     // <= kLocalMaxPieces
  const int cap = kLocalCap / P;
  // A (the row's list has kLocalCap slots, so all of them can be read)
  const int s0 = kMergeSlots * tid;
  uint2 x[kMergeSlots];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.cand + (int64_t)row * kLocalCap + s0);
#pragma unroll
    for (int j = 0; j < kMergeSlots / 2; ++j) {
      const u32x4 q = src[j];
      x[2 * j] = make_uint2(q.x, q.y);
      x[2 * j + 1] = make_uint2(q.z, q.w);
    }
  }
  const uint4 e = tid < P ? a.local[(int64_t)row * a.local_stride + tid] : make_uint4(0u, 0u, 0xFFFFFFFFu, 0u);
  static_assert(kMergeBins == kFT, "one histogram bin per thread to clear");
  hist[tid] = 0u;
  if (tid == 0) sh_short = 0;
  if (tid < P) kept[tid] = (int)e.x;
  const int n_rw = (P + kWave - 1) / kWave;     // waves holding records
  if (wave < n_rw) {
    const uint32_t sum_w = wave_reduce(e.x, [](uint32_t p, uint32_t q) { return p + q; });
    const uint32_t dmax_w = wave_max(e.y), gmin_w = wave_min(e.z), gmax_w = wave_max(e.w);
    if (l == 0) wpart[wave] = make_uint4(sum_w, dmax_w, gmin_w, gmax_w);
  }
  __syncthreads();
  uint32_t m = 0, dmax = 0u, gmin = 0xFFFFFFFFu, gmax = 0u;
  for (int w = 0; w < n_rw; ++w) {
    const uint4 q = wpart[w];
    m += q.x;
    dmax = max(dmax, q.y);
    gmin = min(gmin, q.z);
    gmax = max(gmax, q.w);
  }
  if ((int)m >= a.k) {
    // slot s0 + u lies in piece c0 (or c0 + 1: cap >= 16 > 8 slots); for
    // s < 2^13 and cap <= 2^13, floor(s / cap) = umulhi(s, floor((2^32 - 1) / cap) + 1).
    // This thread's slots [0, e0) hold piece c0's kept entries and [b1, e1)
    // piece c0 + 1's; the key of every other slot becomes 0, which is below
    // every score's key, so no later test sees it
    const uint32_t mul = 0xFFFFFFFFu / (uint32_t)cap + 1u;
    const int c0 = (int)__umulhi((uint32_t)s0, mul);
    const int j0 = s0 - c0 * cap;
    const int kept0 = c0 < P ? kept[c0] : 0, kept1 = c0 + 1 < P ? kept[c0 + 1] : 0;
    const int e0 = min(max(kept0 - j0, 0), kMergeSlots);
    const int b1 = min(cap - j0, kMergeSlots);
    const int e1 = min(cap - j0 + kept1, kMergeSlots);
    const uint32_t valid = ((1u << e0) - 1u) | (((1u << e1) - 1u) & ~((1u << b1) - 1u));
#pragma unroll
    for (int u = 0; u < kMergeSlots; ++u) x[u].x &= 0u - ((valid >> u) & 1u);
    // B: entries above D into the value histogram over (D, largest kept]
    const float lo = key_value(max(dmax + 1u, gmin));
    const float inv = bin_scale(lo, key_value(gmax), kMergeBins);
    const float c = -lo * inv;
    int bn[kMergeSlots];
    int above = 0;
    auto bin_of = [&](float f) { return min(kMergeBins - 1, max(0, (int)fmaf(f, inv, c))); };
    if (dmax >= 0x80000000u) {          // every entry above D is a positive float: its value is key & 0x7fffffff
#pragma unroll
      for (int u = 0; u < kMergeSlots; ++u) {
        bn[u] = -1;
        if (x[u].x > dmax) {
          bn[u] = bin_of(__uint_as_float(x[u].x & 0x7fffffffu));
          ++above;
          atomicAdd(&hist[bn[u]], 1u);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kMergeSlots; ++u) {
        bn[u] = -1;
        if (x[u].x > dmax) {
          bn[u] = bin_of(key_value(x[u].x));
          ++above;
          atomicAdd(&hist[bn[u]], 1u);
        }
      }
    }
    above = (int)wave_reduce((uint32_t)above, [](uint32_t p, uint32_t q) { return p + q; });
    if (l == 0) wabove[wave] = above;
    __syncthreads();
    int n_above = 0;
#pragma unroll
    for (int w = 0; w < kFT / kWave; ++w) n_above += wabove[w];
    if (n_above >= a.k) {
      // C: lane l owns bins 16l .. 16l + 15
      if (wave == 0) {
        uint32_t h[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 q = *reinterpret_cast<const u32x4*>(hist + 16 * l + 4 * j);
          h[4 * j] = q.x; h[4 * j + 1] = q.y; h[4 * j + 2] = q.z; h[4 * j + 3] = q.w;
        }
        uint32_t tot = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) tot += h[j];
        int ab = (int)(wave_suffix_sum(tot) - tot);     // entries in higher lanes' bins
        if (ab < a.k && a.k <= ab + (int)tot) {            // exactly one lane
#pragma unroll
          for (int j = 15; j >= 0; --j) {
            if (ab < a.k && a.k <= ab + (int)h[j]) {
              sel_bin = 16 * l + j;
              sel_above = ab;
            }
            ab += (int)h[j];
          }
        }
      }
      __syncthreads();
      // D
      const int vb = sel_bin, kb = a.k - sel_above;
#pragma unroll
      for (int u = 0; u < kMergeSlots; ++u)
        if (bn[u] == vb) {
          const int j = atomicAdd(&sh_short, 1);
          if (j < kShort) sk[j] = x[u].x;
        }
      __syncthreads();
      const int ns = sh_short;
      if (ns <= kShort) {
        uint32_t v;
        int need;
        if (ns <= kWave) {
          // E: lane i holds short-list key i; v is the key with fewer than kb
          // keys above it and at least kb at or above it
          if (wave == 0) {
            const uint32_t mine = l < ns ? sk[l] : 0u;
            int gt = 0, ge = 0;
            for (int j = 0; j < ns; ++j) {
              const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
              gt += kj > mine;
              ge += kj >= mine;
            }
            const bool hit = l < ns && gt < kb && kb <= ge;
            const uint64_t hm = __ballot(hit);
            if (l == __ffsll((unsigned long long)hm) - 1) {
              sh_v = mine;
              sh_need = kb - gt;
            }
          }
          __syncthreads();
          v = sh_v;
          need = sh_need;
        } else {
          const uint32_t mine = tid < ns ? sk[tid] : 0u;
          const uint32_t bmin = block_reduce<kFT>(tid < ns ? mine : 0xFFFFFFFFu, redu, UMinOp{});
          const uint32_t bmax = block_reduce<kFT>(mine, redu, UMaxOp{});
          v = radix_kth<kFT>(ns, kb, bmin, bmax, [&](int i) { return sk[i]; }, [&](int) { return true; }, hist,
                             &sel_bin, &sel_above, &need);
        }
        // F
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int u = 0; u < kMergeSlots; ++u) {
          gt += x[u].x > v;
          eq += x[u].x == v;
        }
        const uint32_t ex = block_excl_scan1(gt | (eq << 16), wtot);
        int eq_rank = (int)(ex >> 16);
        int out = (int)(ex & 0xFFFFu) + min(eq_rank, need);
#pragma unroll
        for (int u = 0; u < kMergeSlots; ++u) {
          const uint32_t key = x[u].x;
          if (key > v || (key == v && eq_rank++ < need)) {
            if (out < a.k) dst[out] = (int)x[u].y;
            ++out;
          }
        }
        return;
      }
    }
  }
  select_row_single(a.scores + (int64_t)row * a.ld, n, a.k, dst);
}

int64_t chunks_per_row(int64_t max_n) { return (max_n + kChunk - 1) / kChunk; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the few-rows select: the five-pass state (range partials,
// chunk histograms, chunk offsets, row records), the candidate list and the
// standalone pieces' records.
struct TopkLayout {
  float2* rng_own;
  uint32_t* hist;
  int32_t* off;
  RowSel* sel;
  uint2* cand;
  uint4* local;
  int G, PL;
  size_t bytes;
};

TopkLayout topk_layout(void* ws, int rows, int64_t max_n) {
  TopkLayout t{};
  t.G = (int)chunks_per_row(max_n);
  t.PL = (int)((max_n + kLocalSpan - 1) / kLocalSpan);
  const uintptr_t base = reinterpret_cast<uintptr_t>(ws);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const uintptr_t at = base + o;
    o += align256(bytes);
    return at;
  };
  t.rng_own = reinterpret_cast<float2*>(take((size_t)rows * t.G * sizeof(float2)));
  t.hist = reinterpret_cast<uint32_t*>(take((size_t)rows * t.G * kVB * 4));
  t.off = reinterpret_cast<int32_t*>(take((size_t)rows * t.G * 4));
  t.sel = reinterpret_cast<RowSel*>(take((size_t)rows * sizeof(RowSel)));
  t.cand = reinterpret_cast<uint2*>(take((size_t)rows * kCap * sizeof(uint2)));
  t.local = reinterpret_cast<uint4*>(take((size_t)rows * t.PL * sizeof(uint4)));
  t.bytes = o;
  return t;
}

}  // namespace

size_t topk_rows_ws_bytes(int rows, int64_t max_n, int k) {
  if (rows >= kMultiRowLimit || max_n <= k) return 0;
  return topk_layout(nullptr, rows, max_n).bytes;
}

bool topk_rows_local_fits(int rows, int64_t max_n, int k, int span) {
  return topk_rows_ws_bytes(rows, max_n, k) != 0 && (max_n + span - 1) / span <= kLocalMaxPieces;
}

uint2* topk_rows_cand(void* ws, int rows, int64_t max_n) { return topk_layout(ws, rows, max_n).cand; }

hipError_t launch_topk_rows(const float* scores, int64_t ld, int32_t* idx, int rows, int n_q,
                            int64_t q_start, const int64_t* seq_q_start, int k, void* ws, hipStream_t s,
                            const float2* rng, int rng_span, int rng_stride, const uint4* pre_local,
                            int pre_span, int pre_stride) {
  const int64_t max_n = q_start + n_q;
  if (topk_rows_ws_bytes(rows, max_n, k) == 0) {
    hipLaunchKernelGGL(topk_rows_single_kernel, dim3(rows), dim3(kFT), 0, s, scores, ld, idx, n_q,
                       q_start, seq_q_start, k);
    return hipGetLastError();
  }
  if (ws == nullptr) return hipErrorInvalidValue;
  const TopkLayout t = topk_layout(ws, rows, max_n);
  ChunkArgs a{};
  a.scores = scores;
  a.ld = ld;
  a.n_q = n_q;
  a.q_start = q_start;
  a.seq = seq_q_start;
  a.k = k;
  a.G = t.G;
  a.vec = (reinterpret_cast<uintptr_t>(scores) % 16 == 0 && ld % 4 == 0) ? 1 : 0;
  a.rng_own = t.rng_own;
  if (rng) {
    a.rng = rng;
    a.rng_span = rng_span;
    a.rng_stride = rng_stride;
  } else {
    a.rng = a.rng_own;
    a.rng_span = kChunk;
    a.rng_stride = a.G;
  }
  a.hist = t.hist;
  a.off = t.off;
  a.sel = t.sel;
  a.cand = t.cand;
  if (pre_local) {                      // the score kernel ran the wave-local stage
    if ((max_n + pre_span - 1) / pre_span > kLocalMaxPieces) return hipErrorInvalidValue;
    a.local = const_cast<uint4*>(pre_local);
    a.local_span = pre_span;
    a.local_stride = pre_stride;
    hipLaunchKernelGGL(tk_merge_kernel, dim3(rows), dim3(kFT), 0, s, a, idx);
    return hipGetLastError();
  }
  if (t.PL <= kLocalMaxPieces) {
    a.local = t.local;
    a.local_span = kLocalSpan;
    a.local_stride = t.PL;
    hipLaunchKernelGGL(tk_wave_local_kernel, dim3((unsigned)((t.PL + 3) / 4), (unsigned)rows), dim3(256), 0, s,
                       a);
    hipLaunchKernelGGL(tk_merge_kernel, dim3(rows), dim3(kFT), 0, s, a, idx);
    return hipGetLastError();
  }
  const dim3 chunk_grid((unsigned)((int64_t)rows * a.G));
  if (!rng) hipLaunchKernelGGL(tk_range_kernel, chunk_grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(tk_hist_kernel, chunk_grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(tk_select_kernel, dim3(rows), dim3(kST), 0, s, a);
  hipLaunchKernelGGL(tk_collect_kernel, chunk_grid, dim3(kCT), 0, s, a);
  hipLaunchKernelGGL(tk_finish_kernel, dim3(rows), dim3(kFT), 0, s, a, idx);
  return hipGetLastError();
}

}  // namespace ix
