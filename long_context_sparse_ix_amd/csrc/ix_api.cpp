// C ABI of libix: argument validation, workspace sizing, path choice and the
// IndexShare layer-group driver.  All checks run before the first enqueue.
//
// Group schedule ("IndexShare", LLM Architecture Gallery, section "How
// IndexShare Works"; "IndexCache: Killing the Indexer's O(NL^2) Bottleneck"
// notes, section 2): a full layer runs the indexer and top-k and stores the
// positions; a shared layer skips both and attends over the most recent full
// layer's positions; the first layer of a pattern is full.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include "ix.h"
#include "kernels.hpp"

// Scratch of ix_group_forward_noalloc: device memory that exists without any
// allocation call.  Each GPU the library runs on holds its own copy from
// module load until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device address: that comes from
// hipGetSymbolAddress, once per device (scratch_for_stream below).
static __device__ __align__(256) unsigned char scratch[IX_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxK = 2048;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_problem(const ix_problem* p) {
  if (!p) return IX_E_NULL;
  if (p->batch < 1 || p->n_q < 1 || p->q_start < 0 || p->k < 1 || p->k > kMaxK ||
      p->reserved != 0)
    return IX_E_SHAPE;
  if (p->kv_len < p->q_start + p->n_q || p->kv_cap < p->kv_len) return IX_E_SHAPE;
  if (p->kv_len > (int64_t)INT32_MAX) return IX_E_SHAPE;   // positions are int32
  if ((reinterpret_cast<uintptr_t>(p->seq_q_start) & 7u) != 0) return IX_E_SHAPE;
  return IX_OK;
}

int32_t check_indexer(const ix_problem* p, const ix_indexer_in* in) {
  if (!in) return IX_E_NULL;
  if (in->k_dtype != IX_DTYPE_BF16 && in->k_dtype != IX_DTYPE_FP8_E4M3FN) return IX_E_DTYPE;
  if (!in->q || !in->w || !in->k) return IX_E_NULL;
  if (in->k_dtype == IX_DTYPE_FP8_E4M3FN && !in->k_scale) return IX_E_NULL;
  if (in->k_dtype == IX_DTYPE_BF16 && in->k_scale) return IX_E_SHAPE;
  if (in->q_dtype != 0 && in->q_dtype != IX_DTYPE_BF16 && in->q_dtype != IX_DTYPE_FP8_E4M3FN) return IX_E_DTYPE;
  if (in->reserved != 0) return IX_E_SHAPE;
  if (in->q_dtype == IX_DTYPE_FP8_E4M3FN && !in->q_scale) return IX_E_NULL;
  if (in->q_dtype != IX_DTYPE_FP8_E4M3FN && in->q_scale) return IX_E_SHAPE;
  if (in->heads < 1 || in->heads > 64 || in->dim < 16 || in->dim > 128 || in->dim % 16 != 0)
    return IX_E_SHAPE;
  if (in->path < IX_PATH_AUTO || in->path > IX_PATH_MATERIALIZED) return IX_E_SHAPE;
  if (in->path == IX_PATH_FUSED && !ix::fused_dim_supported(in->dim)) return IX_E_SHAPE;
  if (!aligned16(in->q) || !aligned16(in->w) || !aligned16(in->k) ||
      (in->k_scale && !aligned16(in->k_scale)) || (in->q_scale && !aligned16(in->q_scale)))
    return IX_E_SHAPE;
  (void)p;
  return IX_OK;
}

// fp8 queries and fp8 keys with d in {64, 128}: the fused kernel multiplies
// the codes on the fp8 MFMA, reading the key cache in place (no staging).
bool fp8_mma(const ix_indexer_in* in) {
  return in->q_dtype == IX_DTYPE_FP8_E4M3FN && in->k_dtype == IX_DTYPE_FP8_E4M3FN &&
         (in->dim == 64 || in->dim == 128);
}

int32_t check_attn(const ix_attn_in* in) {
  if (!in) return IX_E_NULL;
  if (!in->q || !in->kv || !in->out) return IX_E_NULL;
  if (in->q_heads < 1 || in->q_heads > 16 || !ix::attn_shape_supported(in->d_qk, in->d_v))
    return IX_E_SHAPE;
  if (in->kv_splits < 0 || in->kv_splits > 64 || in->reserved != 0) return IX_E_SHAPE;
  if (!std::isfinite(in->sm_scale)) return IX_E_SHAPE;
  if (!aligned16(in->q) || !aligned16(in->kv) || !aligned16(in->out) ||
      (in->lse && !aligned16(in->lse)))
    return IX_E_SHAPE;
  return IX_OK;
}

bool use_fused(const ix_problem* p, const ix_indexer_in* in) {
  if (in->path == IX_PATH_FUSED) return true;
  if (in->path == IX_PATH_MATERIALIZED || !ix::fused_dim_supported(in->dim)) return false;
  const int64_t rows = (int64_t)p->batch * p->n_q;
  const int64_t score_bytes = rows * p->kv_len * 4;
  return rows >= 128 || score_bytes > ((int64_t)1 << 30);
}

// Fused path: per-row candidate buffers, then (fp8 keys) a bf16 copy of the
// keys any query can reach.  Materialised path: one fp32 score row per query.
size_t fused_cand_bytes(const ix_problem* p) {
  return round_up((size_t)p->batch * p->n_q * (size_t)ix::fused_candidates(p->k) * 8);
}

// Materialised path: fp32 score rows with a 16-byte aligned row stride, then
// the row top-k's own state.
int64_t score_ld(const ix_problem* p) { return (p->kv_len + 3) & ~(int64_t)3; }
size_t score_bytes(const ix_problem* p) {
  return round_up((size_t)p->batch * p->n_q * (size_t)score_ld(p) * 4);
}
size_t topk_ws(const ix_problem* p) {
  return round_up(ix::topk_rows_ws_bytes(p->batch * p->n_q, p->q_start + p->n_q, p->k));
}
// per-wave records of the score kernel for the row select: a (min, max) score
// range, or the wave-local top-k stage's 16-byte record
int rng_stride(const ix_problem* p) { return (int)((p->q_start + p->n_q + ix::kScoreSpan - 1) / ix::kScoreSpan); }
size_t rng_bytes(const ix_problem* p) {
  return round_up((size_t)p->batch * p->n_q * rng_stride(p) * 16);
}

size_t stage_key_bytes(const ix_problem* p, const ix_indexer_in* in) {
  if (fp8_mma(in)) return 0;
  return round_up((size_t)p->batch * (size_t)(p->kv_len + ix::kStagePad) * in->dim * 2);
}
size_t stage_scale_bytes(const ix_problem* p, const ix_indexer_in* in) {
  return in->k_dtype == IX_DTYPE_FP8_E4M3FN && !fp8_mma(in)
             ? round_up((size_t)p->batch * (size_t)(p->kv_len + ix::kStagePad) * 4)
             : 0;
}

size_t argmax_ws(const ix_problem* p, const ix_indexer_in* in) {
  return stage_key_bytes(p, in) + stage_scale_bytes(p, in);
}

size_t indexer_ws(const ix_problem* p, const ix_indexer_in* in) {
  if (use_fused(p, in)) return fused_cand_bytes(p) + stage_key_bytes(p, in) + stage_scale_bytes(p, in);
  return score_bytes(p) + rng_bytes(p) + topk_ws(p);
}

// Work split of the attention.  Many rows: one wave per row.  Few rows: four
// waves share every (row, split) and merge in LDS, and the k slots of a row are
// cut into enough splits for about 1024 waves, each with >= 64 slots; the
// splits' partials are merged by a second kernel.
struct AttnPlan {
  int splits, slots_per_split, wpi;
};

AttnPlan attn_plan(const ix_problem* p, const ix_attn_in* in) {
  const int64_t rows = (int64_t)p->batch * p->n_q;
  AttnPlan pl{};
  pl.wpi = rows < 1024 ? 4 : 1;
  int64_t s = in->kv_splits;
  if (s <= 0) {
    s = pl.wpi == 1 ? 1 : (1024 + rows * 4 - 1) / (rows * 4);
    const int64_t by_slots = p->k / (64 * pl.wpi);
    if (s > by_slots) s = by_slots;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
  }
  const int64_t steps = (p->k + 15) / 16;                  // 16-slot steps
  const int64_t per_wave = (steps + s * pl.wpi - 1) / (s * pl.wpi);
  pl.slots_per_split = (int)(per_wave * 16 * pl.wpi);
  pl.splits = (int)((p->k + pl.slots_per_split - 1) / pl.slots_per_split);   // none empty, <= s
  return pl;
}

size_t attn_ws(const ix_problem* p, const ix_attn_in* in) {
  const int s = attn_plan(p, in).splits;
  if (s <= 1) return 0;
  const size_t items = (size_t)p->batch * p->n_q * s * 16;
  return round_up(items * in->d_v * 4) + round_up(items * 2 * 4);
}

int32_t hip_fail(hipError_t e) {
  g_last_error = hipGetErrorString(e);
  return IX_E_HIP;
}

// Fills the fused kernel's key fields: in the fp8 MFMA form the key cache
// itself; otherwise staged, padded copies of the keys (widened to bf16) and
// fp8 scales at `stage`.
hipError_t stage_fused_keys(const ix_problem* p, const ix_indexer_in* in, char* stage, ix::FusedArgs& a,
                            hipStream_t s) {
  if (fp8_mma(in)) {
    a.keys8 = static_cast<const uint8_t*>(in->k);
    a.key_bstride = p->kv_cap * in->dim;
    a.scale = in->k_scale;
    a.scale_bstride = p->kv_cap;
    a.kv_rows = p->kv_cap;
    return hipSuccess;
  }
  const bool fp8 = in->k_dtype == IX_DTYPE_FP8_E4M3FN;
  const int64_t rows_pad = p->kv_len + ix::kStagePad;
  uint16_t* kb = reinterpret_cast<uint16_t*>(stage);
  float* sb = fp8 ? reinterpret_cast<float*>(stage + stage_key_bytes(p, in)) : nullptr;
  a.keys = kb;
  a.key_bstride = rows_pad * in->dim;
  a.scale = sb;
  a.scale_bstride = fp8 ? rows_pad : 0;
  a.kv_rows = rows_pad;
  return ix::launch_stage_keys(in->k, fp8, p->kv_cap * in->dim, in->k_scale, p->kv_cap, kb, sb, p->batch,
                               p->kv_len, rows_pad, in->dim, s);
}

ix::FusedArgs fused_args(const ix_problem* p, const ix_indexer_in* in, int32_t* idx) {
  ix::FusedArgs a{};
  const bool q8 = in->q_dtype == IX_DTYPE_FP8_E4M3FN;
  a.q = q8 ? nullptr : static_cast<const uint16_t*>(in->q);
  a.q8 = q8 ? static_cast<const uint8_t*>(in->q) : nullptr;
  a.q_scale = q8 ? in->q_scale : nullptr;
  a.w = in->w;
  a.idx = idx;
  a.q_start = p->q_start;
  a.seq_q_start = p->seq_q_start;
  a.n_q = p->n_q;
  a.H = in->heads;
  a.k = p->k;
  return a;
}

int32_t run_indexer(const ix_problem* p, const ix_indexer_in* in, int32_t* idx, void* ws,
                    hipStream_t s) {
  const bool fp8 = in->k_dtype == IX_DTYPE_FP8_E4M3FN;
  if (use_fused(p, in)) {
    ix::FusedArgs a = fused_args(p, in, idx);
    a.C = ix::fused_candidates(p->k);
    a.cand = static_cast<float2*>(ws);
    hipError_t e = stage_fused_keys(p, in, static_cast<char*>(ws) + fused_cand_bytes(p), a, s);
    if (e != hipSuccess) return hip_fail(e);
    e = ix::launch_fused_indexer(a, p->batch, in->dim, s);
    return e == hipSuccess ? IX_OK : hip_fail(e);
  }
  ix::ScoreArgs a{};
  const bool q8 = in->q_dtype == IX_DTYPE_FP8_E4M3FN;
  a.q = q8 ? nullptr : static_cast<const uint16_t*>(in->q);
  a.q8 = q8 ? static_cast<const uint8_t*>(in->q) : nullptr;
  a.q_scale = q8 ? in->q_scale : nullptr;
  a.w = in->w;
  a.keys = in->k;
  a.scale = in->k_scale;
  a.scores = static_cast<float*>(ws);
  a.key_bstride = p->kv_cap * in->dim;
  a.scale_bstride = p->kv_cap;
  a.ld = score_ld(p);
  a.q_start = p->q_start;
  a.seq_q_start = p->seq_q_start;
  a.n_q = p->n_q;
  a.H = in->heads;
  // per-wave records after the scores: (min, max) ranges for the chunked
  // row select, or the wave-local top-k stage's records when it applies
  const int rows = p->batch * p->n_q;
  const int64_t max_n = p->q_start + p->n_q;
  void* per_wave = static_cast<char*>(ws) + score_bytes(p);
  void* tws = static_cast<char*>(ws) + score_bytes(p) + rng_bytes(p);
  const bool local = ix::topk_rows_local_fits(rows, max_n, p->k, ix::kScoreSpan);
  a.rng = local ? nullptr : static_cast<float2*>(per_wave);
  a.local = local ? static_cast<uint4*>(per_wave) : nullptr;
  a.cand = local ? ix::topk_rows_cand(tws, rows, max_n) : nullptr;
  a.rng_stride = rng_stride(p);
  hipError_t e = ix::launch_indexer_scores(a, p->batch, in->dim, fp8, p->kv_len, s);
  if (e != hipSuccess) return hip_fail(e);
  e = ix::launch_topk_rows(a.scores, a.ld, idx, rows, p->n_q, p->q_start, p->seq_q_start, p->k, tws, s, a.rng,
                           ix::kScoreSpan, a.rng_stride, a.local, ix::kScoreSpan, a.rng_stride);
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

// One attention layer.  chain == nullptr: its split partials (if any) are
// merged by a kernel of their own right after it.  Otherwise *chain holds an
// earlier layer's partials still to be merged (splits == 0: none): they are
// merged in this launch's prologue when it runs four waves per (row, split),
// else by their own kernel first; and this layer's partials are left in
// *chain for a later launch (the caller flushes the last with
// ix::launch_attn_combine).
int32_t run_attn(const ix_problem* p, const ix_attn_in* in, const int32_t* idx, void* ws,
                 hipStream_t s, ix::CombineArgs* chain = nullptr) {
  ix::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(in->q);
  a.kv = static_cast<const uint16_t*>(in->kv);
  a.idx = idx;
  a.out = static_cast<uint16_t*>(in->out);
  a.lse = in->lse;
  a.kv_bstride = p->kv_cap * in->d_qk;
  a.kv_len = p->kv_len;
  a.rows = p->batch * p->n_q;
  a.n_q = p->n_q;
  a.Hq = in->q_heads;
  a.k = p->k;
  const AttnPlan pl = attn_plan(p, in);
  a.splits = pl.splits;
  a.slots_per_split = pl.slots_per_split;
  a.wpi = pl.wpi;
  const float sm = in->sm_scale > 0.0f ? in->sm_scale : 1.0f / std::sqrt((float)in->d_qk);
  a.scale_log2 = sm * 1.4426950408889634f;
  if (a.splits > 1) {
    const size_t items = (size_t)a.rows * a.splits * 16;
    a.part_o = static_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(items * in->d_v * 4));
  }
  hipError_t e = hipSuccess;
  if (chain && chain->splits > 1) {
    if (a.wpi > 1) a.prev = *chain;
    else e = ix::launch_attn_combine(*chain, s);
    chain->splits = 0;
    if (e != hipSuccess) return hip_fail(e);
  }
  const bool defer = chain && a.splits > 1;
  e = ix::launch_sparse_attn(a, in->d_qk, in->d_v, s, defer);
  if (e != hipSuccess) return hip_fail(e);
  if (defer) *chain = ix::CombineArgs{a.part_o, a.part_ml, a.out, a.lse, a.rows, a.Hq, a.splits, in->d_v};
  return IX_OK;
}

int32_t check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return IX_OK;
  if (ws_bytes < need) return IX_E_WORKSPACE;
  if (!ws) return IX_E_NULL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return IX_E_SHAPE;
  return IX_OK;
}

// The group's attention layers keep their split partials in two alternating
// halves of this size (a layer's partials are merged by the next layer's
// launch, which writes its own into the other half).
size_t group_attn_half(const ix_problem* p, int32_t n_layers, const ix_attn_in* attn) {
  size_t half = 0;
  for (int l = 0; l < n_layers; ++l) {
    const size_t w = attn_ws(p, &attn[l]);
    if (w > half) half = w;
  }
  return half;
}

size_t group_ws(const ix_problem* p, int32_t n_layers, uint64_t f_mask, const ix_indexer_in* ixr,
                const ix_attn_in* attn) {
  size_t need = 2 * group_attn_half(p, n_layers, attn);
  for (int l = 0; l < n_layers; ++l) {
    if ((f_mask >> l) & 1u) {
      const size_t w = indexer_ws(p, &ixr[l]);
      if (w > need) need = w;
    }
  }
  return need;
}

// Device address of `scratch` on the device of `stream` (the current device
// for the NULL stream), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e);
    if (e2 != hipSuccess) return hip_fail(e2);
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return IX_OK;
}

// Layers of a validated group in order on one stream, workspace ws.
int32_t run_group(const ix_problem* p, int32_t n_layers, uint64_t f_mask, const ix_indexer_in* ixr,
                  const ix_attn_in* attn, int32_t* idx, void* ws, hipStream_t s);

int32_t check_group(const ix_problem* p, int32_t n_layers, uint64_t f_mask,
                    const ix_indexer_in* ixr, const ix_attn_in* attn) {
  if (n_layers < 1 || n_layers > 64) return IX_E_ROLES;
  if (!(f_mask & 1u)) return IX_E_ROLES;
  if (n_layers < 64 && (f_mask >> n_layers) != 0) return IX_E_ROLES;
  if (!ixr || !attn) return IX_E_NULL;
  for (int l = 0; l < n_layers; ++l) {
    if ((f_mask >> l) & 1u) {
      int32_t st = check_indexer(p, &ixr[l]);
      if (st != IX_OK) return st;
    }
    int32_t st = check_attn(&attn[l]);
    if (st != IX_OK) return st;
  }
  return IX_OK;
}

}  // namespace

extern "C" {

int32_t ix_abi_version(void) { return IX_ABI_VERSION; }

const char* ix_status_str(int32_t st) {
  switch (st) {
    case IX_OK: return "IX_OK";
    case IX_E_NULL: return "IX_E_NULL: a required pointer is NULL";
    case IX_E_SHAPE: return "IX_E_SHAPE: unsupported or inconsistent size, or misaligned pointer";
    case IX_E_DTYPE: return "IX_E_DTYPE: unknown key dtype";
    case IX_E_ROLES: return "IX_E_ROLES: bad layer count or role mask (layer 0 must be full)";
    case IX_E_WORKSPACE: return "IX_E_WORKSPACE: workspace too small";
    case IX_E_HIP: return "IX_E_HIP: a HIP launch failed";
    default: return "unknown ix_status";
  }
}

const char* ix_last_error(void) { return g_last_error.c_str(); }

size_t ix_workspace_bytes(const ix_problem* p, int32_t op, const void* desc) {
  if (check_problem(p) != IX_OK) return 0;
  switch (op) {
    case IX_OP_INDEXER_TOPK: {
      auto in = static_cast<const ix_indexer_in*>(desc);
      return check_indexer(p, in) == IX_OK ? indexer_ws(p, in) : 0;
    }
    case IX_OP_SPARSE_ATTN: {
      auto in = static_cast<const ix_attn_in*>(desc);
      return check_attn(in) == IX_OK ? attn_ws(p, in) : 0;
    }
    case IX_OP_GROUP_FORWARD: {
      auto g = static_cast<const ix_group_desc*>(desc);
      if (!g || check_group(p, g->n_layers, g->f_mask, g->ixr, g->attn) != IX_OK) return 0;
      return group_ws(p, g->n_layers, g->f_mask, g->ixr, g->attn);
    }
    case IX_OP_TOPK_SCORES:
      return topk_ws(p);
    case IX_OP_INDEXER_ARGMAX: {
      auto in = static_cast<const ix_indexer_in*>(desc);
      return check_indexer(p, in) == IX_OK && ix::fused_dim_supported(in->dim) ? argmax_ws(p, in) : 0;
    }
    default:
      return 0;
  }
}

int32_t ix_indexer_topk(const ix_problem* p, const ix_indexer_in* in, int32_t* idx, void* ws,
                        size_t ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st == IX_OK) st = check_indexer(p, in);
  if (st != IX_OK) return st;
  if (!idx) return IX_E_NULL;
  if (!aligned16(idx)) return IX_E_SHAPE;
  st = check_ws(indexer_ws(p, in), ws, ws_bytes);
  if (st != IX_OK) return st;
  return run_indexer(p, in, idx, ws, static_cast<hipStream_t>(stream));
}

int32_t ix_indexer_argmax(const ix_problem* p, const ix_indexer_in* in, int32_t* pos, float* score, void* ws,
                          size_t ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st == IX_OK) st = check_indexer(p, in);
  if (st != IX_OK) return st;
  if (!pos) return IX_E_NULL;
  if (!ix::fused_dim_supported(in->dim) || in->path == IX_PATH_MATERIALIZED) return IX_E_SHAPE;
  if ((reinterpret_cast<uintptr_t>(pos) & 3u) != 0 || (reinterpret_cast<uintptr_t>(score) & 3u) != 0)
    return IX_E_SHAPE;
  st = check_ws(argmax_ws(p, in), ws, ws_bytes);
  if (st != IX_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ix::FusedArgs a = fused_args(p, in, pos);
  a.best = score;
  hipError_t e = stage_fused_keys(p, in, static_cast<char*>(ws), a, s);
  if (e != hipSuccess) return hip_fail(e);
  e = ix::launch_fused_argmax(a, p->batch, in->dim, s);
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

int32_t ix_sparse_attn(const ix_problem* p, const ix_attn_in* in, const int32_t* idx, void* ws,
                       size_t ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st == IX_OK) st = check_attn(in);
  if (st != IX_OK) return st;
  if (!idx) return IX_E_NULL;
  if (!aligned16(idx)) return IX_E_SHAPE;
  st = check_ws(attn_ws(p, in), ws, ws_bytes);
  if (st != IX_OK) return st;
  return run_attn(p, in, idx, ws, static_cast<hipStream_t>(stream));
}

int32_t ix_group_forward(const ix_problem* p, int32_t n_layers, uint64_t f_mask,
                         const ix_indexer_in* ixr, const ix_attn_in* attn, int32_t* idx,
                         void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st == IX_OK) st = check_group(p, n_layers, f_mask, ixr, attn);
  if (st != IX_OK) return st;
  if (!idx) return IX_E_NULL;
  if (!aligned16(idx)) return IX_E_SHAPE;
  st = check_ws(group_ws(p, n_layers, f_mask, ixr, attn), ws, ws_bytes);
  if (st != IX_OK) return st;
  return run_group(p, n_layers, f_mask, ixr, attn, idx, ws, static_cast<hipStream_t>(stream));
}

int32_t ix_group_forward_noalloc(const ix_problem* p, int32_t n_layers, uint64_t f_mask,
                                 const ix_indexer_in* ixr, const ix_attn_in* attn, int32_t* idx, void* stream) {
  int32_t st = check_problem(p);
  if (st == IX_OK) st = check_group(p, n_layers, f_mask, ixr, attn);
  if (st != IX_OK) return st;
  if (!idx) return IX_E_NULL;
  if (!aligned16(idx)) return IX_E_SHAPE;
  const size_t need = group_ws(p, n_layers, f_mask, ixr, attn);
  if (need > (size_t)IX_NOALLOC_SCRATCH_BYTES) {
    g_last_error = "ix_group_forward_noalloc: the call needs " + std::to_string(need) +
                   " bytes of scratch, the static scratch holds " +
                   std::to_string((size_t)IX_NOALLOC_SCRATCH_BYTES);
    return IX_E_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_for_stream(s, &ws)) != IX_OK) return st;
  return run_group(p, n_layers, f_mask, ixr, attn, idx, ws, s);
}

int32_t ix_topk_scores(const ix_problem* p, const float* scores, int64_t ld, int32_t* idx,
                       void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_problem(p);
  if (st != IX_OK) return st;
  if (!scores || !idx) return IX_E_NULL;
  if (ld < p->kv_len || !aligned16(scores) || !aligned16(idx)) return IX_E_SHAPE;
  st = check_ws(topk_ws(p), ws, ws_bytes);
  if (st != IX_OK) return st;
  hipError_t e = ix::launch_topk_rows(scores, ld, idx, p->batch * p->n_q, p->n_q, p->q_start, p->seq_q_start,
                                      p->k, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

int32_t ix_index_overlap(const ix_problem* p, const int32_t* idx_a, const int32_t* idx_b, int32_t* counts,
                         void* stream) {
  int32_t st = check_problem(p);
  if (st != IX_OK) return st;
  if (!idx_a || !idx_b || !counts) return IX_E_NULL;
  if (!aligned16(idx_a) || !aligned16(idx_b) || (reinterpret_cast<uintptr_t>(counts) & 3u) != 0)
    return IX_E_SHAPE;
  hipError_t e = ix::launch_index_overlap(idx_a, idx_b, counts, (int64_t)p->batch * p->n_q, p->k,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

int32_t ix_append_keys(const ix_problem* p, int32_t dim, const float* k_new, int32_t n_new, int64_t pos,
                       uint8_t* k_cache, float* k_scale, void* stream) {
  int32_t st = check_problem(p);
  if (st != IX_OK) return st;
  if (!k_new || !k_cache || !k_scale) return IX_E_NULL;
  if (dim < 16 || dim > 128 || dim % 16 != 0 || n_new < 0 || pos < 0 || pos + n_new > p->kv_cap)
    return IX_E_SHAPE;
  if (p->seq_q_start && pos < p->q_start) return IX_E_SHAPE;   // keeps every shifted row >= 0
  if (!aligned16(k_new) || !aligned16(k_cache) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0)
    return IX_E_SHAPE;
  hipError_t e = ix::launch_append_keys(k_new, k_cache, k_scale, p->batch, n_new, pos, p->seq_q_start,
                                        p->q_start, p->kv_cap, dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

int32_t ix_indexer_project(int64_t rows, const ix_project_in* in, void* q_out, float* w_out, void* stream) {
  if (!in || !in->x || !in->w_proj || !q_out || !w_out) return IX_E_NULL;
  if (rows < 0 || in->heads < 1 || in->dim < 1 || in->d_in < 64 || in->d_in % 64 != 0 || in->reserved != 0)
    return IX_E_SHAPE;
  const int64_t n = (int64_t)in->heads * in->dim + in->heads;
  if (n >= (int64_t)INT32_MAX) return IX_E_SHAPE;
  // a 256-row tile of x or W spans < 2^31 bytes; the 64 x 64 tile count fits an int
  if (in->d_in >= (1 << 22) || ((rows + 63) / 64) * ((n + 63) / 64) > (int64_t)INT32_MAX) return IX_E_SHAPE;
  if (!aligned16(in->x) || !aligned16(in->w_proj) || (reinterpret_cast<uintptr_t>(q_out) & 1u) != 0 ||
      (reinterpret_cast<uintptr_t>(w_out) & 3u) != 0)
    return IX_E_SHAPE;
  ix::ProjArgs a{};
  a.x = static_cast<const uint16_t*>(in->x);
  a.w = static_cast<const uint16_t*>(in->w_proj);
  a.q = static_cast<uint16_t*>(q_out);
  a.wo = w_out;
  a.M = rows;
  a.N = (int)n;
  a.K = in->d_in;
  a.Nq = in->heads * in->dim;
  hipError_t e = ix::launch_indexer_project(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

int32_t ix_quantize_queries(int64_t n_rows, int32_t dim, const void* q, uint8_t* codes, float* scale,
                            void* stream) {
  if (!q || !codes || !scale) return IX_E_NULL;
  if (n_rows < 0 || dim < 16 || dim > 128 || dim % 16 != 0 || n_rows > ((int64_t)1 << 54)) return IX_E_SHAPE;
  if (!aligned16(q) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scale) & 3u) != 0) return IX_E_SHAPE;
  hipError_t e = ix::launch_quantize_queries(static_cast<const uint16_t*>(q), codes, scale, n_rows, dim,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? IX_OK : hip_fail(e);
}

}  // extern "C"

namespace {

int32_t run_group(const ix_problem* p, int32_t n_layers, uint64_t f_mask, const ix_indexer_in* ixr,
                  const ix_attn_in* attn, int32_t* idx, void* ws, hipStream_t s) {
  const size_t slot = (size_t)p->batch * p->n_q * p->k;
  const size_t half = group_attn_half(p, n_layers, attn);
  int32_t* cur = nullptr;
  int f = 0;
  ix::CombineArgs pending{};           // the previous layer's partials, merged by the next launch
  for (int l = 0; l < n_layers; ++l) {
    if ((f_mask >> l) & 1u) {          // full layer: fresh positions into its own slot
      if (pending.splits > 1) {        // the indexer's workspace overlaps the partials
        hipError_t e = ix::launch_attn_combine(pending, s);
        pending.splits = 0;
        if (e != hipSuccess) return hip_fail(e);
      }
      cur = idx + slot * f++;
      const int32_t st = run_indexer(p, &ixr[l], cur, ws, s);
      if (st != IX_OK) return st;
    }
    // shared layers reuse `cur` untouched
    const int32_t st = run_attn(p, &attn[l], cur, static_cast<char*>(ws) + (l & 1) * half, s, &pending);
    if (st != IX_OK) return st;
  }
  if (pending.splits > 1) {
    hipError_t e = ix::launch_attn_combine(pending, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return IX_OK;
}

}  // namespace
