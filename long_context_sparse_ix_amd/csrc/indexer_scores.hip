// Indexer scores written out as fp32 rows (few-row workloads such as decode).
//
// Same score as the fused kernel ("IndexShare", LLM Architecture Gallery,
// section "Why The Indexer Becomes Expensive"):
//     score(p, s) = sum_h w[h] * max(0, q[h,:] . key[s,:]),  s <= p,
// but for workloads with only a handful of query rows (decode: one row per
// sequence) there is nothing to share across rows, so the key range of every
// row is split over many waves instead and each wave streams its own keys
// from HBM into MFMA B operands.  fp8 keys of width 128 load coalesced (1 KB
// per instruction) and pass through a small wave-private LDS transpose;
// other widths load each lane's key directly.  fp8 e4m3fn keys are widened
// to bf16 in registers (exact) and the per-key scale is applied to the
// finished score.  The row's head weights sit in LDS, shared by the
// workgroup's four waves.  The rows are then reduced by the per-row top-k: for rows of
// at most 512 waves' spans, each wave first keeps the best of its own 640
// scores for the row's candidate list (the top-k's wave-local stage, run here
// as the epilogue on the scores just written), so the top-k itself is one
// merge pass.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "topk_local.hpp"

namespace ix {

namespace {

constexpr int kTileKeys = 64;
constexpr int kTilesPerWave = kScoreSpan / kTileKeys;   // 10 tiles of 64 keys per wave
constexpr int kWavesPerWG = 4;

template <int HT, int KS, bool FP8>
__global__ __launch_bounds__(kWavesPerWG * kWave, FP8 ? 2 : 1) void indexer_scores_kernel(ScoreArgs a) {
  constexpr int d = KS * 16;
  // tiles per wave held in registers (one in use, the rest in flight).  fp8
  // keys: one tile ahead, which leaves room for two waves per SIMD (one
  // computes while the other waits on its keys; measured faster than one
  // wave with four tiles ahead); bf16 tiles are twice the bytes, so one wave
  // per SIMD with two tiles ahead.
  constexpr int kDepth = FP8 ? 2 : 3;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int m = l & 31, hf = l >> 5;
  const int row = blockIdx.y;                 // b * n_q + t
  const int b = row / a.n_q, t = row % a.n_q;
  const int64_t p = seq_start(a.seq_q_start, b, a.q_start) + t;
  const int64_t s_begin = ((int64_t)blockIdx.x * kWavesPerWG + wave) * kTilesPerWave * kTileKeys;
  // The row's head weights sit in LDS (all four waves score the same row)
  // rather than in 32 registers per lane.  Filled before any wave leaves.
  __shared__ __align__(16) float w_lds[HT * 32];
  for (int i = threadIdx.x; i < HT * 32; i += kWavesPerWG * kWave)
    w_lds[i] = i < a.H ? a.w[(int64_t)row * a.H + i] * (a.q_scale ? a.q_scale[(int64_t)row * a.H + i] : 1.0f)
                       : 0.0f;
  __syncthreads();
  if (s_begin > p) return;
  const int n_tiles = (int)min<int64_t>(kTilesPerWave, (p - s_begin) / kTileKeys + 1);

  const float* scale_b = FP8 ? a.scale + (int64_t)b * a.scale_bstride : nullptr;
  float* out = a.scores + (int64_t)row * a.ld;

  // Raw key bytes of one 64-key tile for this lane: key s0 + nt*32 + m, bytes
  // (fp8) or elements (bf16) [hf*d/2, +d/2), plus (fp8) the scale of key
  // s0 + l.  kDepth - 1 tiles are in flight while one is widened and used.
  constexpr int RAW = FP8 ? (KS % 2 == 0 ? KS / 2 : KS) : KS;   // 16-byte (or 8-byte) pieces per half
  typedef typename std::conditional<FP8 && (KS % 2 != 0), u32x2, u32x4>::type piece_t;
  // fp8 keys of d = 128 (128 bytes a key) load coalesced: piece c of half nt
  // is the c-th kilobyte of the half tile's 32 keys (lane l: key 8c + l/8,
  // bytes 16 (l%8) ..), and an LDS transpose gives each lane its key's bytes.
  // Lane-per-key loads touched 32 cache lines per instruction and kept the
  // texture addresser ~87% busy.
  constexpr bool kCoal = FP8 && KS == 8;
  piece_t raw[kDepth][2][RAW];
  float sc[kDepth];
  auto load_raw = [&](int64_t s0, piece_t (&rw)[2][RAW], float& scl) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if constexpr (kCoal) {
        // 32-bit offsets from the wave's (uniform) first key: a wave's span is
        // 640 keys, so they stay small whatever the context length
        const unsigned char* kb = static_cast<const unsigned char*>(a.keys) + (int64_t)b * a.key_bstride + s_begin * d;
        const uint32_t lim = (uint32_t)min<int64_t>((p - s_begin) * d + d - 16, (int64_t)UINT32_MAX);
        const uint32_t off0 = (uint32_t)((s0 - s_begin + nt * 32) * d) + 16u * (uint32_t)l;
#pragma unroll
        for (int c = 0; c < RAW; ++c)   // keys past p read key p's last piece (inside the cache; masked below)
          rw[nt][c] = *reinterpret_cast<const piece_t*>(kb + min(off0 + 1024u * c, lim));
        continue;
      }
      int64_t s = s0 + nt * 32 + m;
      if (s > p) s = p;                       // stays inside the cache; masked below
      const unsigned char* kr = static_cast<const unsigned char*>(a.keys) +
                                ((int64_t)b * a.key_bstride + s * d + hf * (d / 2)) * (FP8 ? 1 : 2);
#pragma unroll
      for (int c = 0; c < RAW; ++c) rw[nt][c] = *reinterpret_cast<const piece_t*>(kr + c * sizeof(piece_t));
    }
    if constexpr (FP8) scl = scale_b[min<int64_t>(s0 + l, p)];
  };
  auto widen = [&](const piece_t (&rw)[RAW], bf16x8 (&bfr)[KS]) {
    if constexpr (FP8 && KS % 2 == 0) {
#pragma unroll
      for (int c = 0; c < KS / 2; ++c) {
        const u32x4 v = rw[c];
        const u32x2 r0 = e4m3x4_to_bf16x4(v.x), r1 = e4m3x4_to_bf16x4(v.y);
        const u32x2 r2 = e4m3x4_to_bf16x4(v.z), r3 = e4m3x4_to_bf16x4(v.w);
        bfr[2 * c] = __builtin_bit_cast(bf16x8, u32x4{r0.x, r0.y, r1.x, r1.y});
        bfr[2 * c + 1] = __builtin_bit_cast(bf16x8, u32x4{r2.x, r2.y, r3.x, r3.y});
      }
    } else if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const u32x2 v = rw[c];
        const u32x2 r0 = e4m3x4_to_bf16x4(v.x), r1 = e4m3x4_to_bf16x4(v.y);
        bfr[c] = __builtin_bit_cast(bf16x8, u32x4{r0.x, r0.y, r1.x, r1.y});
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bfr[ks] = __builtin_bit_cast(bf16x8, rw[ks]);
    }
  };

  // fp8 queries: e4m3fn codes widened exactly to bf16 (their per-head scale
  // is folded into the head weight above)
  bf16x8 qf[HT][KS];
  if (a.q8) {
    const uint8_t* qrow = a.q8 + (int64_t)row * a.H * d;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + m;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < a.H) {
          const u32x2 c = *reinterpret_cast<const u32x2*>(qrow + (int64_t)h * d + hf * (d / 2) + 8 * ks);
          const u32x2 lo = e4m3x4_to_bf16x4(c.x), hi = e4m3x4_to_bf16x4(c.y);
          v = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        qf[ht][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  } else {
    const uint16_t* qrow = a.q + (int64_t)row * a.H * d;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 32 + m;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ht][ks] = h < a.H ? *reinterpret_cast<const bf16x8*>(qrow + (int64_t)h * d + hf * (d / 2) + 8 * ks)
                             : bf16x8{};
    }
  }

  // Loads are unconditional (keys past p are clamped to p, their scores are
  // masked): exec-masked load branches make the compiler's memory-counter
  // waits drain every load in flight, the prefetched tiles included.
#pragma unroll
  for (int j = 0; j < kDepth - 1; ++j) load_raw(s_begin + (int64_t)j * kTileKeys, raw[j], sc[j]);

  // kCoal transpose buffer, private to the wave: key r's 16-byte piece c sits
  // in slot c ^ ((r >> 1) & 7) of its 128-byte row, so both the stores (two
  // keys per 16 lanes) and the reads (16 keys per 16 lanes) fall in distinct
  // banks.
  __shared__ __align__(16) u32x4 tbuf[kWavesPerWG][kCoal ? 512 : 1];
  u32x4* const tb = tbuf[wave];
  auto park_tile = [&](const piece_t (&rw)[2][RAW]) {
    if constexpr (kCoal) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int c = 0; c < RAW; ++c) {
          const int r = 8 * c + (l >> 3);
          tb[nt * 256 + r * 8 + ((l & 7) ^ ((r >> 1) & 7))] = rw[nt][c];
        }
      wave_lds_sync();                         // this wave's stores, then other lanes' reads
    }
  };
  // this lane's key (m) bytes [64 hf, +64) of half nt, from the parked tile
  auto half_pieces = [&](int nt, piece_t (&pc)[RAW]) {
    if constexpr (kCoal) {
#pragma unroll
      for (int cc = 0; cc < RAW; ++cc) pc[cc] = tb[nt * 256 + m * 8 + ((4 * hf + cc) ^ ((m >> 1) & 7))];
    }
  };

  float smin = INFINITY, smax = -INFINITY;     // range of this wave's scores
  float kept[kTilesPerWave] = {};               // this lane's score of every tile (top-k stage)
  // fully unrolled, so `kept` stays in registers; a partial last group
  // computes masked tiles
#pragma unroll
  for (int j0 = 0; j0 < kTilesPerWave; j0 += kDepth) {
    if (j0 >= n_tiles) break;
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int j = j0 + u;
      {
        const int jn = j + kDepth - 1;
        load_raw(s_begin + (int64_t)jn * kTileKeys, raw[(u + kDepth - 1) % kDepth], sc[(u + kDepth - 1) % kDepth]);
        const int64_t s0 = s_begin + (int64_t)j * kTileKeys;
        park_tile(raw[u]);
        // the two 32-key halves one after the other: only one half's B
        // fragments and accumulators are live, which leaves room for two
        // waves per SIMD (one computes while the other waits on its keys)
        float part[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          bf16x8 bfr[KS];
          if constexpr (kCoal) {
            piece_t pc[RAW];
            half_pieces(nt, pc);
            widen(pc, bfr);
          } else {
            widen(raw[u][nt], bfr);
          }
          f32x16 acc[HT];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
              acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ht][ks], bfr[ks], ks == 0 ? f32x16{} : acc[ht],
                                                                0, 0, 0);
          float sacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              // weights of heads ht*32 + 8 r4 + 4 hf + (0..3): accumulator
              // rows 4 r4 .. 4 r4 + 3 of this lane
              const f32x4 wv = *reinterpret_cast<const f32x4*>(w_lds + ht * 32 + 8 * r4 + 4 * hf);
#pragma unroll
              for (int i = 0; i < 4; ++i) sacc[i] = fmaf(wv[i], relu(acc[ht][4 * r4 + i]), sacc[i]);
            }
          part[nt] = (sacc[0] + sacc[1]) + (sacc[2] + sacc[3]);
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                         __float_as_uint(part[1]), false, false);
        float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int64_t s = s0 + l;
        // (a partial last group of bf16's three-tile groups runs past the
        // wave's ten tiles; those scores are masked and not kept)
        if (j < kTilesPerWave) kept[j < kTilesPerWave ? j : 0] = FP8 ? score * sc[u] : score;
        if (s <= p) {
          if constexpr (FP8) score *= sc[u];
          out[(uint32_t)s] = score;             // 32-bit index off a wave-uniform base
          smin = fminf(smin, score);
          smax = fmaxf(smax, score);
        }
      }
    }
  }
  if (a.local) {
    // wave-local top-k stage over this wave's scores (entries past p, and
    // tiles past the last, are masked)
    const int piece = blockIdx.x * kWavesPerWG + wave;
    const int P = (int)((p + kScoreSpan) / kScoreSpan);       // waves that score this row
    // keys s_begin .. p are valid (at most kScoreSpan of them are this wave's)
    const int64_t rem64 = p + 1 - s_begin;
    const int rem = rem64 < 0 ? 0 : (rem64 > kScoreSpan ? kScoreSpan : (int)rem64);
    const int cap = kLocalCap / P;
    __shared__ uint32_t hist[kWavesPerWG][kLocalBins];
    const uint4 r = wave_keep_top<kTilesPerWave>(kept, rem, (int)s_begin, cap, hist[wave],
                                                 a.cand + (int64_t)row * kLocalCap + (int64_t)piece * cap);
    if (l == 0) a.local[(int64_t)row * a.rng_stride + piece] = r;
  } else if (a.rng) {
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) {
      smin = fminf(smin, __shfl_xor(smin, dd));
      smax = fmaxf(smax, __shfl_xor(smax, dd));
    }
    if (l == 0) a.rng[(int64_t)row * a.rng_stride + blockIdx.x * kWavesPerWG + wave] = make_float2(smin, smax);
  }
}

template <int HT, int KS, bool FP8>
hipError_t launch_scores_t(const ScoreArgs& a, int B, int64_t kv_len, hipStream_t st) {
  const int64_t keys_per_wg = (int64_t)kWavesPerWG * kTilesPerWave * kTileKeys;
  const int64_t max_keys = a.q_start + a.n_q;   // last row sees this many keys
  (void)kv_len;
  dim3 grid((unsigned)((max_keys + keys_per_wg - 1) / keys_per_wg), (unsigned)(B * a.n_q));
  hipLaunchKernelGGL((indexer_scores_kernel<HT, KS, FP8>), grid, dim3(kWavesPerWG * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const ScoreArgs& a, int B, int d, bool fp8, int64_t kv_len,
                                 hipStream_t s) {
  const int HT = a.H > 32 ? 2 : 1;
  const int KS = d / 16;
#define IX_SC_CASE(ht, ks)                                                   \
  if (HT == ht && KS == ks)                                                  \
    return fp8 ? launch_scores_t<ht, ks, true>(a, B, kv_len, s)              \
               : launch_scores_t<ht, ks, false>(a, B, kv_len, s);
  IX_SC_CASE(1, 1) IX_SC_CASE(1, 2) IX_SC_CASE(1, 3) IX_SC_CASE(1, 4)
  IX_SC_CASE(1, 5) IX_SC_CASE(1, 6) IX_SC_CASE(1, 7) IX_SC_CASE(1, 8)
  IX_SC_CASE(2, 1) IX_SC_CASE(2, 2) IX_SC_CASE(2, 3) IX_SC_CASE(2, 4)
  IX_SC_CASE(2, 5) IX_SC_CASE(2, 6) IX_SC_CASE(2, 7) IX_SC_CASE(2, 8)
#undef IX_SC_CASE
  return hipErrorInvalidValue;
}

}  // namespace ix
