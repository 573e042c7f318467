/*
 * ix.h -- C ABI of the MI355X (gfx950) DSA layer-group library "libix".
 *
 * The method (DeepSeek Sparse Attention under GLM-5.2's IndexShare schedule):
 *   - "IndexShare" (LLM Architecture Gallery), section "Why The Indexer
 *     Becomes Expensive": a lightweight indexer scores the tokens preceding a
 *     query and keeps the top-k positions; the main attention then runs over
 *     that subset only.
 *   - "GLM-5.2 and IndexShare for Long-Context Sparse Attention", section
 *     "Where the DSA indexer becomes expensive": k = 2,048.
 *   - "IndexShare", section "How IndexShare Works": a full (F) layer runs the
 *     indexer and the top-k and stores the selected positions; a shared (S)
 *     layer skips both and reuses the most recent F layer's positions; only
 *     those integer positions are shared.
 *   - "IndexCache: Killing the Indexer's O(NL^2) Bottleneck" notes, section 2:
 *     the first layer of a pattern is always F.
 *
 * Conventions for every entry point
 *   - Tensors are row-major, last dimension innermost.  "B" is the number of
 *     independent sequences, "n_q" query rows per sequence, "cap" the row
 *     stride of the per-sequence key / latent-KV caches.
 *   - Query row t of a sequence sits at absolute position p = q_start + t and
 *     may select any key position s with 0 <= s <= p (itself included).
 *     q_start + n_q <= kv_len <= kv_cap is required.
 *   - Sequences of different lengths (serving batches): with
 *     ix_problem.seq_q_start set, row t of sequence b sits at
 *     p = seq_q_start[b] + t instead, and q_start is the largest start, which
 *     sizes the launches and the workspace.  A sequence's keys past its own
 *     last row are never read, so its valid length needs no array of its own;
 *     kv_len stays the common bound.
 *   - All pointers except the problem/descriptor structs are DEVICE pointers
 *     (HBM of the current HIP device) and must be 16-byte aligned.  The
 *     caller allocates and owns every buffer, including the workspace; the
 *     library allocates no device memory and keeps no pointer after a call
 *     returns.  Buffers must stay alive until the work on `stream` completes.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they enqueue kernels and return.
 *   - Every argument is validated before anything is enqueued: a non-IX_OK
 *     return means nothing was launched.  IX_E_HIP reports a failed launch;
 *     ix_last_error() then holds the HIP error text.  No C++ exception
 *     crosses the ABI.  Calls on one stream are ordered; the library holds no
 *     global mutable state besides the last-error string, so different
 *     streams/threads may call concurrently.
 */
#ifndef IX_H_
#define IX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IX_ABI_VERSION 7

typedef enum ix_status {
  IX_OK = 0,
  IX_E_NULL = 1,       /* a required pointer is NULL                         */
  IX_E_SHAPE = 2,      /* unsupported or inconsistent size, or misalignment  */
  IX_E_DTYPE = 3,      /* unknown key dtype                                   */
  IX_E_ROLES = 4,      /* n_layers outside [1, 64], or layer 0 is not F       */
  IX_E_WORKSPACE = 5,  /* ws_bytes smaller than ix_workspace_bytes()          */
  IX_E_HIP = 6         /* a HIP launch failed                                 */
} ix_status;

typedef enum ix_dtype {
  IX_DTYPE_BF16 = 1,        /* bfloat16 values                                 */
  IX_DTYPE_FP8_E4M3FN = 2   /* OCP FP8 E4M3FN codes times a per-row fp32 scale */
} ix_dtype;

typedef enum ix_indexer_path {
  IX_PATH_AUTO = 0,         /* library picks: fused when there are many rows   */
  IX_PATH_FUSED = 1,        /* scores streamed straight into the top-k, never stored;
                               needs dim in {16, 32, 64, 128} (else IX_E_SHAPE) */
  IX_PATH_MATERIALIZED = 2  /* one fp32 score row per query in the workspace, then top-k */
} ix_indexer_path;

typedef enum ix_op {
  IX_OP_INDEXER_TOPK = 1,   /* op_desc: const ix_indexer_in*  */
  IX_OP_SPARSE_ATTN = 2,    /* op_desc: const ix_attn_in*     */
  IX_OP_GROUP_FORWARD = 3,  /* op_desc: const ix_group_desc*  */
  IX_OP_TOPK_SCORES = 4,    /* op_desc: NULL                  */
  IX_OP_INDEXER_ARGMAX = 5  /* op_desc: const ix_indexer_in*  */
} ix_op;

/* Sizes shared by every layer of a call. */
typedef struct ix_problem {
  int32_t batch;    /* B >= 1                                                  */
  int32_t n_q;      /* query rows per sequence, >= 1                           */
  int64_t q_start;  /* absolute position of query row 0, >= 0                  */
  int64_t kv_len;   /* valid key rows per sequence, q_start + n_q <= kv_len    */
  int64_t kv_cap;   /* allocated rows per sequence (row stride), >= kv_len     */
  int32_t k;        /* positions kept per query row, 1 <= k <= 2048            */
  int32_t reserved; /* must be 0                                               */
  /* NULL (every sequence starts at q_start), or a DEVICE array int64 [batch]
   * (8-byte aligned) of per-sequence starts, each in [0, q_start]; q_start is
   * then their maximum or any larger value that keeps q_start + n_q <= kv_len.
   * The values are read by the kernels, not by the host: an entry outside
   * [0, q_start] is clamped into it (its sequence's result is then that of the
   * clamped start; memory accesses stay inside the buffers either way).  Used
   * by ix_indexer_topk, ix_group_forward (full layers), ix_topk_scores and
   * ix_append_keys; attention reads positions from idx only. */
  const int64_t* seq_q_start;
} ix_problem;

/* Inputs of one full layer's indexer.
 * score(t, s) = sum_h w[t,h] * max(0, q[t,h,:] . key[s,:]), where key[s,:] is
 * the bf16 row, or the e4m3fn codes of row s times k_scale[s].  The pages
 * describe the indexer only as a small low-rank FP8 module with few heads
 * (IndexCache notes, section 1); this weighted-ReLU form is the library's
 * stated reading.  Queries are bf16 by default; with q_dtype
 * IX_DTYPE_FP8_E4M3FN they are e4m3fn codes times one fp32 scale per (row,
 * head), q[t,h,:] = codes[t,h,:] * q_scale[t,h] (a mode the caller declares;
 * ix_quantize_queries makes them from bf16 queries).  With FP8 keys and d in
 * {64, 128} the fused kernel then multiplies the codes on fp8 MFMA and reads
 * the key cache in place; otherwise the codes are widened exactly to bf16.
 * The scales factor out of the ReLU, so k_scale and q_scale must be >= 0 (as
 * max|x|/448 scales are); a negative or NaN scale gives unspecified scores
 * (memory accesses stay inside the buffers). */
typedef struct ix_indexer_in {
  int32_t heads;    /* H, 1..64                                                */
  int32_t dim;      /* d, a multiple of 16 in 16..128                          */
  int32_t k_dtype;  /* ix_dtype of `k`                                         */
  int32_t path;     /* ix_indexer_path                                         */
  const void* q;    /* [B][n_q][H][d]: bf16, or uint8 e4m3fn codes (q_dtype)   */
  const float* w;   /* fp32 [B][n_q][H]                                        */
  const void* k;    /* [B][kv_cap][d]: bf16, or uint8 e4m3fn codes             */
  const float* k_scale; /* fp32 [B][kv_cap] for FP8 keys; must be NULL for bf16 */
  int32_t q_dtype;  /* 0 or IX_DTYPE_BF16: bf16 q; IX_DTYPE_FP8_E4M3FN: e4m3fn codes */
  int32_t reserved; /* must be 0                                               */
  const float* q_scale; /* fp32 [B][n_q][H], 16-byte aligned, for FP8 queries;
                           must be NULL for bf16 queries                       */
} ix_indexer_in;

/* Inputs/outputs of one layer's sparse attention over selected latent rows.
 * o[t,h,:] = sum_j softmax_j(sm_scale * q[t,h,:] . kv[idx_j,:]) * kv[idx_j,:d_v]
 * over the slots j of row t whose idx lies in [0, kv_len) (others ignored). */
typedef struct ix_attn_in {
  int32_t q_heads;  /* Hq, 1..16                                               */
  int32_t d_qk;     /* D: latent row width (key = whole row); 128 or 576       */
  int32_t d_v;      /* Dv: value = first Dv dims; 96/128 for D=128, 512 for D=576 */
  float sm_scale;   /* softmax scale; <= 0 selects 1/sqrt(D)                  */
  int32_t kv_splits;/* slot-range splits per row (0 = library choice), <= 64   */
  int32_t reserved; /* must be 0                                               */
  const void* q;    /* bf16 [B][n_q][Hq][D]                                    */
  const void* kv;   /* bf16 [B][kv_cap][D]                                     */
  void* out;        /* bf16 [B][n_q][Hq][Dv]                                   */
  float* lse;       /* optional fp32 [B][n_q][Hq]: natural-log sum of exp(logits); -inf for an empty row */
} ix_attn_in;

/* A layer group, for ix_workspace_bytes(IX_OP_GROUP_FORWARD). */
typedef struct ix_group_desc {
  int32_t n_layers;
  int32_t reserved;
  uint64_t f_mask;
  const ix_indexer_in* ixr;   /* host array [n_layers] */
  const ix_attn_in* attn;     /* host array [n_layers] */
} ix_group_desc;

int32_t ix_abi_version(void);
const char* ix_status_str(int32_t status);
/* Text of the last IX_E_HIP failure on the calling thread, or of the last
 * IX_E_WORKSPACE rejection by ix_group_forward_noalloc ("" if none). */
const char* ix_last_error(void);

/* Workspace bytes `op` needs for `prob` and its descriptor (0 if none).
 * Returns 0 also when the arguments are invalid; the entry point then reports
 * the precise status. */
size_t ix_workspace_bytes(const ix_problem* prob, int32_t op, const void* op_desc);

/* Full-layer indexer and top-k (one F layer).
 * Passages: "IndexShare" (LLM Architecture Gallery), section "Why The Indexer
 * Becomes Expensive" -- the indexer scores every preceding token of a query
 * and the top-k positions are kept; "GLM-5.2 and IndexShare for Long-Context
 * Sparse Attention", section "Where the DSA indexer becomes expensive" --
 * k = 2,048 per query position; "IndexShare", section "How IndexShare Works"
 * -- a full layer runs this step and stores the positions.
 * Writes idx int32 [B][n_q][k]: for each query row, the min(k, p+1) positions
 * with the largest scores (equal scores: lower position wins), in ascending
 * position order, then -1 up to k.  The fp32 score matrix is never stored on
 * the fused path (scores stream straight into a per-row candidate set).
 * Workspace: ix_workspace_bytes(prob, IX_OP_INDEXER_TOPK, in) bytes, 256-byte
 * aligned, caller-owned, contents undefined on entry and on return.
 * Errors: IX_E_NULL / IX_E_SHAPE / IX_E_DTYPE for bad arguments,
 * IX_E_WORKSPACE when ws_bytes is too small, IX_E_HIP for a failed launch. */
int32_t ix_indexer_topk(const ix_problem* prob, const ix_indexer_in* in, int32_t* idx,
                        void* ws, size_t ws_bytes, void* stream);

/* Top-1 of the same indexer scores: for each query row, the position with the
 * largest score (equal scores: lower position) into pos int32 [B][n_q] and,
 * if score is not NULL, that fp32 score into score [B][n_q].  This is
 * ix_indexer_topk with k = 1 under the same rule ("IndexShare", LLM
 * Architecture Gallery, section "Why The Indexer Becomes Expensive"), run by
 * the fused kernel with a running maximum in place of the streaming top-k, so
 * its time is the score stream's alone.  Fused path only: dim in {16, 32,
 * 64, 128} and in->path not IX_PATH_MATERIALIZED, else IX_E_SHAPE.  prob->k
 * is validated but unused.  pos and score 4-byte aligned.  Workspace:
 * ix_workspace_bytes(prob, IX_OP_INDEXER_ARGMAX, in) bytes (the staged keys). */
int32_t ix_indexer_argmax(const ix_problem* prob, const ix_indexer_in* in, int32_t* pos, float* score,
                          void* ws, size_t ws_bytes, void* stream);

/* Sparse attention of one layer over an index buffer idx int32 [B][n_q][k]
 * (typically written by ix_indexer_topk).
 * Passages: "IndexShare" (LLM Architecture Gallery), section "Why The Indexer
 * Becomes Expensive" -- the main attention runs only over the selected
 * subset; "GLM-5.2 and IndexShare for Long-Context Sparse Attention", section
 * "What IndexShare reuses" -- every layer, shared or not, computes its own
 * attention over the shared positions.
 * Entries outside [0, kv_len) are ignored; latent rows outside [0, kv_len)
 * are never read.  out (and lse if given) are written for every row; a row
 * with no valid entry gets o = 0 and lse = -inf.  Workspace:
 * ix_workspace_bytes(prob, IX_OP_SPARSE_ATTN, in) bytes (0 when rows are many:
 * split partials only exist for few rows).  Errors as ix_indexer_topk. */
int32_t ix_sparse_attn(const ix_problem* prob, const ix_attn_in* in, const int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream);

/* One IndexShare layer group, layers run in order on `stream`.
 * Passages: "IndexShare" (LLM Architecture Gallery), section "How IndexShare
 * Works" -- full layers compute and store positions, shared layers skip the
 * indexer and top-k and reuse the nearest preceding full layer's integer
 * positions; "IndexCache: Killing the Indexer's O(NL^2) Bottleneck" notes,
 * section 2 -- the first layer of a pattern is full; "GLM-5.2 and IndexShare
 * for Long-Context Sparse Attention", section "What IndexShare reuses" -- the
 * released pattern repeats full, shared, shared, shared after a few initial
 * exceptions, which any f_mask expresses.
 * Bit l of f_mask set => layer l is full (F): it runs ix_indexer_topk with
 * ixr[l] into the next slot of idx, then attends; clear => shared (S): it
 * attends over the most recent F layer's slot, byte for byte unchanged.
 * Bit 0 must be set and 1 <= n_layers <= 64.  ixr entries of S layers are
 * ignored (may be zeroed).  idx: int32 [popcount(f_mask & ((1<<n)-1))][B][n_q][k]. */
int32_t ix_group_forward(const ix_problem* prob, int32_t n_layers, uint64_t f_mask,
                         const ix_indexer_in* ixr, const ix_attn_in* attn, int32_t* idx,
                         void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch ix_group_forward_noalloc works in. */
#define IX_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* ix_group_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * (a decode step is one group call), harnesses that forbid hipMalloc.  Same
 * arguments, semantics and results (byte for byte) as ix_group_forward, whose
 * kernels it runs; their workspace is instead a file-scope static __device__
 * array of IX_NOALLOC_SCRATCH_BYTES (64 MiB) in the library, of which each
 * GPU the library runs on holds one copy from load until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the first call on a device looks up that device's scratch
 * address once (hipGetSymbolAddress, with the stream's device current).
 * A call whose workspace would exceed the scratch -- ix_workspace_bytes(prob,
 * IX_OP_GROUP_FORWARD, desc) > IX_NOALLOC_SCRATCH_BYTES, e.g. long prefills
 * on the fused path -- returns IX_E_WORKSPACE before anything is enqueued,
 * with the sizes in ix_last_error().  Every call on one GPU shares that GPU's
 * scratch and its contents stay from the last call (no kernel of the group
 * needs them zeroed: each writes its scratch before reading it); calls that
 * overlap on one GPU -- concurrent streams, or threads -- race on it, so the
 * caller must order them (e.g. one stream).  Other errors as
 * ix_group_forward. */
int32_t ix_group_forward_noalloc(const ix_problem* prob, int32_t n_layers, uint64_t f_mask,
                                 const ix_indexer_in* ixr, const ix_attn_in* attn, int32_t* idx,
                                 void* stream);

/* The top-k step alone, over caller-provided fp32 score rows (the selection
 * of "IndexShare" (LLM Architecture Gallery), section "How IndexShare Works",
 * with k as in "GLM-5.2 and IndexShare for Long-Context Sparse Attention",
 * section "Where the DSA indexer becomes expensive"): scores[(b*n_q + t)*ld + s] for
 * s <= p = q_start + t, or seq_q_start[b] + t (entries beyond p are ignored).  Same selection rule
 * and output layout as ix_indexer_topk.  ld >= kv_len.  Scores must not be
 * NaN.  Calls with few long rows (B*n_q < 1024 and q_start + n_q > k) keep
 * their select state in ws, of ix_workspace_bytes(prob, IX_OP_TOPK_SCORES,
 * NULL) bytes; other calls need none (ws may be NULL). */
int32_t ix_topk_scores(const ix_problem* prob, const float* scores, int64_t ld, int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream);

/* Per-row overlap of two index buffers: counts[b*n_q + t] = the number of
 * positions present in both idx_a[b][t][:] and idx_b[b][t][:], negative slots
 * ignored.  It measures the adjacent-layer overlap that makes index reuse
 * work ("IndexShare", LLM Architecture Gallery, section "Why Reusing Indices
 * Can Work").  idx_a, idx_b: int32 [B][n_q][k] in the layout ix_indexer_topk
 * writes (ascending valid positions, then -1; another layout gives an
 * unspecified count but no access outside the rows); counts: int32 [B][n_q].
 * Only batch, n_q and k of prob are used (prob is still validated).  Needs no
 * workspace; IX_E_NULL on a NULL pointer, IX_E_SHAPE on misaligned idx
 * buffers. */
int32_t ix_index_overlap(const ix_problem* prob, const int32_t* idx_a, const int32_t* idx_b,
                         int32_t* counts, void* stream);

/* New indexer keys into the fp8 key cache (the cache format ix_indexer_topk
 * reads with k_dtype IX_DTYPE_FP8_E4M3FN; the pages store indexer keys in FP8,
 * IndexCache notes, section 1).  For every sequence b and new row r < n_new,
 * with x = k_new[(b*n_new + r)*dim + j] (fp32):
 *   scale = max_j |x_j| / 448 (1 for an all-zero row), correctly rounded fp32;
 *   code_j = e4m3fn(x_j / scale): correctly rounded fp32 quotient, then round
 *            to nearest with ties to the even code, saturating at +-448;
 * codes go to k_cache[(b*kv_cap + pos_b + r)*dim + j] and the scale to
 * k_scale[b*kv_cap + pos_b + r], where pos_b = pos, or, with
 * prob->seq_q_start set, pos_b = pos - q_start + seq_q_start[b] (the entry
 * clamped into [0, q_start] as everywhere): each sequence's rows move down by
 * its distance below the largest start, so pos = q_start appends the new
 * token of a decode step at every sequence's own position.  Other cache rows
 * are untouched.  Uses batch, q_start, seq_q_start and kv_cap of prob (prob
 * is still validated).  dim: a multiple of 16 in 16..128; n_new >= 0;
 * 0 <= pos and pos + n_new <= kv_cap, and pos >= q_start when seq_q_start is
 * set.  k_new 16-byte aligned, k_scale 4-byte aligned.  No workspace.
 * IX_E_NULL on a NULL pointer, IX_E_SHAPE on a bad size or alignment. */
int32_t ix_append_keys(const ix_problem* prob, int32_t dim, const float* k_new, int32_t n_new, int64_t pos,
                       uint8_t* k_cache, float* k_scale, void* stream);

/* Indexer inputs from hidden states.  The pages describe the indexer as a
 * small low-rank module with few heads (IndexCache notes, section 1); this
 * library's reading is one bf16 input row per query and one bf16 weight:
 *   y[r][n] = sum_j x[r][j] * w_proj[n][j]   (fp32 accumulation),
 *   q_out[r][h][i] = bf16(y[r][h*dim + i])   (nearest, ties to even),
 *   w_out[r][h]    = y[r][heads*dim + h]     (fp32),
 * i.e. the q and w arguments of ix_indexer_topk for these rows. */
typedef struct ix_project_in {
  int32_t heads;          /* H >= 1                                           */
  int32_t dim;            /* d >= 1                                           */
  int32_t d_in;           /* input width, a multiple of 64 in [64, 2^22)      */
  int32_t reserved;       /* must be 0                                        */
  const void* x;          /* bf16 [rows][d_in], 16-byte aligned               */
  const void* w_proj;     /* bf16 [heads*dim + heads][d_in], 16-byte aligned  */
} ix_project_in;

/* Computes q_out (bf16 [rows][heads][dim], 2-byte aligned) and w_out (fp32
 * [rows][heads], 4-byte aligned) from in (see above).  rows >= 0 (0 does
 * nothing); heads*dim + heads < 2^31; ceil(rows/64) * ceil((heads*dim +
 * heads)/64) < 2^31.  Caller-owned buffers, no workspace.
 * IX_E_NULL on a NULL pointer, IX_E_SHAPE on a bad size, a nonzero reserved
 * field or misalignment, IX_E_HIP on a launch failure. */
int32_t ix_indexer_project(int64_t rows, const ix_project_in* in, void* q_out, float* w_out, void* stream);

/* Indexer queries into the declared fp8 form (ix_indexer_in.q_dtype =
 * IX_DTYPE_FP8_E4M3FN).  The pages make the indexer a small FP8 module
 * (IndexCache notes, section 1); the per-(row, head) scaling is the library's
 * reading, the same as the key cache's (see ix_append_keys): for every row r
 * of dim bf16 values q[r][:] (a row is one query row's head, so n_rows =
 * B*n_q*H for an indexer q of [B][n_q][H][dim]),
 *   scale[r]    = max_j |q[r][j]| / 448, or 1 for an all-zero row,
 *   codes[r][j] = e4m3fn(q[r][j] / scale[r]),
 * rounded to nearest with ties to the even code and saturating at +-448, both
 * divisions correctly rounded fp32 (a negative value that rounds to zero
 * keeps its sign bit).  q: bf16 [n_rows][dim], 16-byte aligned; codes: uint8
 * [n_rows][dim], 16-byte aligned; scale: fp32 [n_rows], 4-byte aligned; all
 * caller-owned, no workspace.  dim a multiple of 16 in [16, 128]; n_rows >= 0
 * (0 does nothing).  IX_E_NULL on a NULL pointer, IX_E_SHAPE on a bad size or
 * misalignment, IX_E_HIP on a launch failure. */
int32_t ix_quantize_queries(int64_t n_rows, int32_t dim, const void* q, uint8_t* codes, float* scale,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IX_H_ */
