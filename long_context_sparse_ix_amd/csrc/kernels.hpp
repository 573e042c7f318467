// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ix {

// Fused indexer score + streaming top-k (prefill and chunked prefill).
struct FusedArgs {
  const uint16_t* q;      // bf16 [B][n_q][H][d], or nullptr when q8 is set
  const uint8_t* q8;      // e4m3fn codes [B][n_q][H][d], or nullptr
  const float* q_scale;   // with q8: fp32 [B][n_q][H], the codes' scale
  const float* w;         // [B][n_q][H]
  const uint16_t* keys;   // bf16 rows, row stride d, sequence stride key_bstride
  const uint8_t* keys8;   // or e4m3fn code rows read in place (fp8 MFMA form; needs q8,
                          // scale and d in {64, 128}); key_bstride then counts bytes
  const float* scale;     // per-key fp32 scale, or nullptr
  int64_t kv_rows;        // key rows that exist per sequence (tile loads past them read zeros)
  int32_t* idx;           // [B][n_q][k]; the argmax variant: [B][n_q] best positions
  float* best;            // argmax variant: [B][n_q] best scores (nullable)
  float2* cand;           // workspace: per row C fp32 scores then C int32 positions (C float2 of room)
  int64_t key_bstride;    // elements
  int64_t scale_bstride;  // elements
  int64_t q_start;        // row 0's position (with seq_q_start: the largest start)
  const int64_t* seq_q_start;   // nullable: per-sequence start of row 0 [B]
  int n_q, H, k, C;       // C: candidate slots per row (>= k + 64)
};
size_t fused_lds_bytes(int d);
bool fused_dim_supported(int d);   // d in {16, 32, 64, 128}
int fused_candidates(int k);
hipError_t launch_fused_indexer(const FusedArgs& a, int B, int d, hipStream_t s);
// The same score stream with a running maximum instead of the top-k: idx[row]
// = the row's best position (equal scores: lower), best[row] = its score.
// Uses neither cand nor C nor k.
hipError_t launch_fused_argmax(const FusedArgs& a, int B, int d, hipStream_t s);

// e4m3fn codes -> bf16 (exact), rows [0, rows) of every sequence.
// Key staging for the fused indexer: the first `rows` key rows of every
// sequence as bf16 (e4m3fn codes widened exactly, or bf16 copied) into
// dst [B][rows_padded][d], and (fp8) their scales into dst_scale
// [B][rows_padded]; rows in [rows, rows_padded) are zero, so whole-tile loads
// never leave the buffer.
hipError_t launch_stage_keys(const void* src, bool fp8, int64_t src_bstride, const float* scale,
                             int64_t scale_bstride, uint16_t* dst, float* dst_scale, int B, int64_t rows,
                             int64_t rows_padded, int d, hipStream_t s);
constexpr int kStagePad = 64;     // rows of padding after the last key (one tile)

// Materialised indexer scores: scores[(b*n_q+t)*ld + s] for s <= q_start+t.
struct ScoreArgs {
  const uint16_t* q;      // bf16 queries, or nullptr when q8 is set
  const uint8_t* q8;      // e4m3fn query codes (widened to bf16 at load), or nullptr
  const float* q_scale;   // with q8: fp32 [rows][H]
  const float* w;
  const void* keys;       // bf16 or e4m3fn codes, row stride d, sequence stride key_bstride
  const float* scale;     // fp8 only
  float* scores;
  int64_t key_bstride;    // elements
  int64_t scale_bstride;
  int64_t ld;
  int64_t q_start;        // row 0's position (with seq_q_start: the largest start)
  const int64_t* seq_q_start;   // nullable: per-sequence start of row 0 [B]
  int n_q, H;
  float2* rng;            // nullable: per-wave (min, max) of the written scores,
                          // [rows][rng_stride], one entry per kScoreSpan keys
  uint4* local;           // nullable (then rng is unused): the wave-local top-k stage runs
                          // as the epilogue, records [rows][rng_stride], kept entries
                          // into cand [rows][8192] (the row top-k's candidate list)
  uint2* cand;
  int rng_stride;
};
constexpr int kScoreSpan = 640;    // keys per wave of the score kernel (10 tiles of 64)
hipError_t launch_indexer_scores(const ScoreArgs& a, int B, int d, bool fp8, int64_t kv_len,
                                 hipStream_t s);

// Per-row top-k over materialised fp32 score rows.  Few rows use
// multi-workgroup selects whose state lives in a workspace of
// topk_rows_ws_bytes(rows, q_start + n_q, k) bytes (0: none needed): a
// wave-local keep stage over pieces of the row plus a per-row merge when a row
// has at most 512 pieces, else five chunked passes.  `rng` (nullable, five-pass
// select only) holds per-row (min, max) partials over consecutive spans of
// rng_span scores, rng_stride entries per row; without it the select measures
// the ranges itself.  `pre_local` (nullable) says the wave-local stage already
// ran over pieces of pre_span positions (the score kernel's epilogue): its
// per-piece records are [rows][pre_stride] and its kept entries are in the
// workspace's candidate list (topk_rows_cand), so only the merge runs.
size_t topk_rows_ws_bytes(int rows, int64_t max_n, int k);
// true when the wave-local stage applies to pieces of `span` positions
bool topk_rows_local_fits(int rows, int64_t max_n, int k, int span);
uint2* topk_rows_cand(void* ws, int rows, int64_t max_n);
// Row r = b * n_q + t holds the candidates 0 .. start_b + t, start_b the
// per-sequence start seq_q_start[b] (clamped into [0, q_start]) or q_start.
hipError_t launch_topk_rows(const float* scores, int64_t ld, int32_t* idx, int rows, int n_q,
                            int64_t q_start, const int64_t* seq_q_start, int k, void* ws, hipStream_t s,
                            const float2* rng = nullptr, int rng_span = 0, int rng_stride = 0,
                            const uint4* pre_local = nullptr, int pre_span = 0, int pre_stride = 0);

// New fp32 key rows [B][n_new][dim] -> e4m3fn codes and fp32 scales at cache
// rows [pos_b, pos_b + n_new) of sequence b (dim a multiple of 16, <= 128):
// pos_b = pos, or with seq_shift, pos - shift_bound + seq_shift[b] (the entry
// clamped into [0, shift_bound]; the caller keeps pos >= shift_bound).
hipError_t launch_append_keys(const float* k_new, uint8_t* k_cache, float* k_scale, int B, int n_new, int64_t pos,
                              const int64_t* seq_shift, int64_t shift_bound, int64_t kv_cap, int dim,
                              hipStream_t s);

// bf16 rows [n_rows][dim] -> e4m3fn codes [n_rows][dim] and one fp32 scale
// per row (max|x|/448, 1 for a zero row); dim a multiple of 16 in [16, 128].
hipError_t launch_quantize_queries(const uint16_t* src, uint8_t* codes, float* scale, int64_t n_rows, int dim,
                                   hipStream_t s);

// Indexer inputs from hidden states: [q | w] = x . W^T with x bf16 [M][K],
// W bf16 [N][K] (K a multiple of 64); the first Nq columns go to q as bf16
// (nearest, ties to even) [M][Nq], the rest to wo as fp32 [M][N - Nq].
struct ProjArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* q;
  float* wo;
  int64_t M;
  int N, K, Nq;
};
hipError_t launch_indexer_project(const ProjArgs& a, hipStream_t s);

// Per-row overlap count of two [rows][k] index buffers (k <= 2048).
hipError_t launch_index_overlap(const int32_t* a, const int32_t* b, int32_t* counts, int64_t rows, int k,
                                hipStream_t s);

// Sparse gather attention.
// Split partials of one attention launch that still have to be merged into
// its output (splits > 1), or none (splits == 0).
struct CombineArgs {
  const float* part_o;    // [rows][splits][16][Dv]
  const float* part_ml;   // [rows][splits][16][2]
  uint16_t* out;          // [rows][Hq][Dv]
  float* lse;             // [rows][Hq] or nullptr
  int rows, Hq, splits, Dv;
};

struct AttnArgs {
  const uint16_t* q;      // [B][n_q][Hq][D]
  const uint16_t* kv;     // [B][cap][D]
  const int32_t* idx;     // [B][n_q][k]
  uint16_t* out;          // [B][n_q][Hq][Dv]
  float* lse;             // [B][n_q][Hq] or nullptr
  float* part_o;          // splits > 1: [rows][splits][16][Dv]
  float* part_ml;         // splits > 1: [rows][splits][16][2]
  int64_t kv_bstride;     // elements
  int64_t kv_len;
  int rows, n_q, Hq, k, splits, slots_per_split;
  int wpi;                // waves per (row, split): 1, or 4 sharing the split's slots
  float scale_log2;       // sm_scale * log2(e)
  CombineArgs prev;       // wpi == 4 only: an earlier launch's partials, merged in this
                          // launch's prologue (prev.splits == 0: none)
};
bool attn_shape_supported(int d_qk, int d_v);
// Launches the attention; with splits > 1 also the merge of its partials,
// unless defer_combine (the caller then merges them later: in a following
// wpi == 4 launch's prologue, or by launch_attn_combine).
hipError_t launch_sparse_attn(const AttnArgs& a, int d_qk, int d_v, hipStream_t s, bool defer_combine = false);
hipError_t launch_attn_combine(const CombineArgs& c, hipStream_t s);

}  // namespace ix
