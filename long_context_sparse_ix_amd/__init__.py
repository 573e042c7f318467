"""MI355X-native DSA layer group under the IndexShare schedule.

Thin Python binding over the C ABI in ``include/ix.h`` (``libix.so``, built
from ``csrc/`` for gfx950).  The functions below only marshal torch tensors
into pointers and sizes; every step of the indexer, the top-k and the sparse
attention runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

The method, as the pages describe it ("IndexShare", LLM Architecture Gallery,
sections "Why The Indexer Becomes Expensive" and "How IndexShare Works"): a
full layer runs a lightweight indexer over every preceding token, keeps the
top-k positions (k = 2,048 in GLM-5.2) and stores them; the next shared layers
skip the indexer and attend over those same positions with their own queries
and latent KV.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import torch

__all__ = [
    "IxError", "ix_abi_version", "ix_status_str", "ix_workspace_bytes", "ix_indexer_topk",
    "ix_sparse_attn", "ix_group_forward", "ix_topk_scores", "ix_index_overlap", "ix_append_keys",
    "ix_indexer_argmax", "ix_group_forward_noalloc", "ix_indexer_project", "ix_quantize_queries",
    "NOALLOC_SCRATCH_BYTES", "lib_path",
    "load",
    "IX_PATH_AUTO", "IX_PATH_FUSED", "IX_PATH_MATERIALIZED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libix.so")

ABI_VERSION = 7
IX_OK, IX_E_NULL, IX_E_SHAPE, IX_E_DTYPE, IX_E_ROLES, IX_E_WORKSPACE, IX_E_HIP = range(7)
IX_DTYPE_BF16, IX_DTYPE_FP8_E4M3FN = 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20          # IX_NOALLOC_SCRATCH_BYTES in ix.h
IX_PATH_AUTO, IX_PATH_FUSED, IX_PATH_MATERIALIZED = 0, 1, 2
IX_OP_INDEXER_TOPK, IX_OP_SPARSE_ATTN, IX_OP_GROUP_FORWARD, IX_OP_TOPK_SCORES, IX_OP_INDEXER_ARGMAX = 1, 2, 3, 4, 5


class Problem(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_q", c_int32), ("q_start", c_int64), ("kv_len", c_int64),
                ("kv_cap", c_int64), ("k", c_int32), ("reserved", c_int32), ("seq_q_start", c_void_p)]


class IndexerIn(ctypes.Structure):
    _fields_ = [("heads", c_int32), ("dim", c_int32), ("k_dtype", c_int32), ("path", c_int32),
                ("q", c_void_p), ("w", c_void_p), ("k", c_void_p), ("k_scale", c_void_p),
                ("q_dtype", c_int32), ("reserved", c_int32), ("q_scale", c_void_p)]


class AttnIn(ctypes.Structure):
    _fields_ = [("q_heads", c_int32), ("d_qk", c_int32), ("d_v", c_int32), ("sm_scale", c_float),
                ("kv_splits", c_int32), ("reserved", c_int32), ("q", c_void_p), ("kv", c_void_p),
                ("out", c_void_p), ("lse", c_void_p)]


class ProjectIn(ctypes.Structure):
    _fields_ = [("heads", c_int32), ("dim", c_int32), ("d_in", c_int32), ("reserved", c_int32),
                ("x", c_void_p), ("w_proj", c_void_p)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("reserved", c_int32), ("f_mask", c_uint64),
                ("ixr", POINTER(IndexerIn)), ("attn", POINTER(AttnIn))]


class IxError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = ""
        if _lib is not None and (status == IX_E_HIP or (status == IX_E_WORKSPACE and what.endswith("_noalloc"))):
            detail = ": " + _lib.ix_last_error().decode()
        super().__init__(f"{what}: {ix_status_str(status)}{detail}")
        self.status = status


_lib = None


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load libix.so (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_sparse_ix_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ix_abi_version.restype = c_int32
    lib.ix_abi_version.argtypes = []
    lib.ix_status_str.restype = ctypes.c_char_p
    lib.ix_status_str.argtypes = [c_int32]
    lib.ix_last_error.restype = ctypes.c_char_p
    lib.ix_last_error.argtypes = []
    lib.ix_workspace_bytes.restype = c_size_t
    lib.ix_workspace_bytes.argtypes = [POINTER(Problem), c_int32, c_void_p]
    lib.ix_indexer_topk.restype = c_int32
    lib.ix_indexer_topk.argtypes = [POINTER(Problem), POINTER(IndexerIn), c_void_p, c_void_p,
                                    c_size_t, c_void_p]
    lib.ix_indexer_argmax.restype = c_int32
    lib.ix_indexer_argmax.argtypes = [POINTER(Problem), POINTER(IndexerIn), c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p]
    lib.ix_sparse_attn.restype = c_int32
    lib.ix_sparse_attn.argtypes = [POINTER(Problem), POINTER(AttnIn), c_void_p, c_void_p, c_size_t,
                                   c_void_p]
    lib.ix_group_forward.restype = c_int32
    lib.ix_group_forward.argtypes = [POINTER(Problem), c_int32, c_uint64, POINTER(IndexerIn),
                                     POINTER(AttnIn), c_void_p, c_void_p, c_size_t, c_void_p]
    lib.ix_group_forward_noalloc.restype = c_int32
    lib.ix_group_forward_noalloc.argtypes = [POINTER(Problem), c_int32, c_uint64, POINTER(IndexerIn),
                                             POINTER(AttnIn), c_void_p, c_void_p]
    lib.ix_topk_scores.restype = c_int32
    lib.ix_topk_scores.argtypes = [POINTER(Problem), c_void_p, c_int64, c_void_p, c_void_p,
                                   c_size_t, c_void_p]
    lib.ix_append_keys.restype = c_int32
    lib.ix_append_keys.argtypes = [POINTER(Problem), c_int32, c_void_p, c_int32, c_int64, c_void_p, c_void_p,
                                   c_void_p]
    lib.ix_index_overlap.restype = c_int32
    lib.ix_index_overlap.argtypes = [POINTER(Problem), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.ix_indexer_project.restype = c_int32
    lib.ix_indexer_project.argtypes = [c_int64, POINTER(ProjectIn), c_void_p, c_void_p, c_void_p]
    lib.ix_quantize_queries.restype = c_int32
    lib.ix_quantize_queries.argtypes = [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    if lib.ix_abi_version() != ABI_VERSION:   # the structs above follow this version of ix.h
        raise ImportError(f"{LIB_PATH} has ABI {lib.ix_abi_version()}, this binding needs {ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def ix_abi_version() -> int:
    return load().ix_abi_version()


def ix_status_str(status: int) -> str:
    return load().ix_status_str(status).decode()


# ---------------------------------------------------------------- helpers --
def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name):
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


_ws_cache: dict = {}


def _torch_stream(stream, device):
    """The torch stream object a call enqueues on (current stream by default)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _workspace(nbytes: int, device, stream=None):
    """A workspace of at least nbytes for calls on (device, stream).  One
    buffer is cached per (device, stream) and allocated on that stream, so
    calls on different streams never share bytes, and when a larger request
    replaces a buffer the caching allocator hands its block out again only
    after the work already queued on that stream."""
    if nbytes == 0:
        return None, 0
    dev = torch.device(device)
    s = _torch_stream(stream, dev)
    key = (dev.index, s.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        _ws_cache.pop(key, None)
        with torch.cuda.stream(s):
            buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf, nbytes


def _problem(batch, n_q, q_start, kv_len, kv_cap, k, seq_q_start=None):
    return Problem(batch, n_q, int(q_start), int(kv_len), int(kv_cap), int(k), 0, _ptr(seq_q_start))


def _starts(seq_q_start, q_start, batch):
    """Checks a per-sequence start array and returns the common bound: the
    given q_start, or (None) the array's maximum, which costs a device sync."""
    if seq_q_start is None:
        return 0 if q_start is None else int(q_start)
    _dev(seq_q_start, "seq_q_start")
    _need(seq_q_start.dtype == torch.int64 and tuple(seq_q_start.shape) == (batch,),
          "seq_q_start must be int64 [B] on the device")
    return int(seq_q_start.max().item()) if q_start is None else int(q_start)


def _key_dtype(keys):
    if keys.dtype == torch.bfloat16:
        return IX_DTYPE_BF16
    if keys.dtype in (torch.uint8, torch.float8_e4m3fn):
        return IX_DTYPE_FP8_E4M3FN
    raise ValueError(f"indexer keys must be bf16 or e4m3fn codes, got {keys.dtype}")


def _indexer_in(q, w, keys, k_scale, path, q_scale=None):
    _dev(q, "q"), _dev(w, "w"), _dev(keys, "keys")
    q8 = q.dtype in (torch.uint8, torch.float8_e4m3fn)
    _need((q.dtype == torch.bfloat16 or q8) and q.dim() == 4,
          "indexer q must be bf16 or e4m3fn codes [B, n_q, H, d]")
    if q8:
        _need(q_scale is not None, "fp8 queries need q_scale [B, n_q, H]")
        _dev(q_scale, "q_scale")
        _need(q_scale.dtype == torch.float32 and tuple(q_scale.shape) == tuple(q.shape[:3]),
              "q_scale must be fp32 [B, n_q, H]")
    else:
        _need(q_scale is None, "bf16 queries take no q_scale")
    _need(w.dtype == torch.float32 and tuple(w.shape) == tuple(q.shape[:3]), "w must be fp32 [B, n_q, H]")
    kd = _key_dtype(keys)
    _need(keys.dim() == 3 and keys.shape[0] == q.shape[0] and keys.shape[2] == q.shape[3],
          "keys must be [B, cap, d]")
    if kd == IX_DTYPE_FP8_E4M3FN:
        _need(k_scale is not None, "fp8 keys need k_scale [B, cap]")
        _dev(k_scale, "k_scale")
        _need(k_scale.dtype == torch.float32 and tuple(k_scale.shape) == tuple(keys.shape[:2]),
              "k_scale must be fp32 [B, cap]")
    else:
        _need(k_scale is None, "bf16 keys take no k_scale")
    return IndexerIn(q.shape[2], q.shape[3], kd, path, _ptr(q), _ptr(w), _ptr(keys), _ptr(k_scale),
                     IX_DTYPE_FP8_E4M3FN if q8 else IX_DTYPE_BF16, 0, _ptr(q_scale))


def _attn_in(q, kv, out, lse, sm_scale, kv_splits):
    _dev(q, "q"), _dev(kv, "kv"), _dev(out, "out")
    _need(q.dtype == torch.bfloat16 and q.dim() == 4, "attention q must be bf16 [B, n_q, Hq, D]")
    _need(kv.dtype == torch.bfloat16 and kv.dim() == 3 and kv.shape[2] == q.shape[3],
          "kv must be bf16 [B, cap, D]")
    _need(out.dtype == torch.bfloat16 and tuple(out.shape[:3]) == tuple(q.shape[:3]),
          "out must be bf16 [B, n_q, Hq, Dv]")
    if lse is not None:
        _dev(lse, "lse")
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == tuple(q.shape[:3]),
              "lse must be fp32 [B, n_q, Hq]")
    return AttnIn(q.shape[2], q.shape[3], out.shape[3], float(sm_scale), int(kv_splits), 0,
                  _ptr(q), _ptr(kv), _ptr(out), _ptr(lse))


def _check(status, what):
    if status != IX_OK:
        raise IxError(status, what)


# ------------------------------------------------------------- entry points --
def ix_workspace_bytes(prob: Problem, op: int, desc) -> int:
    ref = None if desc is None else ctypes.byref(desc)
    return load().ix_workspace_bytes(ctypes.byref(prob), op, ref)


def ix_indexer_topk(q, w, keys, idx, *, k_scale=None, q_start=None, kv_len=None, path=IX_PATH_AUTO,
                    seq_q_start=None, q_scale=None, stream=None):
    """Full-layer indexer + top-k into ``idx`` int32 [B, n_q, k] (see ix.h).

    ``seq_q_start`` (int64 [B] on the device, optional): per-sequence position
    of row 0; ``q_start`` is then their bound (default: their maximum).  With
    ``q`` as e4m3fn codes (uint8), ``q_scale`` fp32 [B, n_q, H] is their scale."""
    lib = load()
    _dev(idx, "idx")
    _need(idx.dtype == torch.int32 and tuple(idx.shape[:2]) == tuple(q.shape[:2]), "idx must be int32 [B, n_q, k]")
    cap = keys.shape[1]
    q_start = _starts(seq_q_start, q_start, q.shape[0])
    prob = _problem(q.shape[0], q.shape[1], q_start, cap if kv_len is None else kv_len, cap, idx.shape[2],
                    seq_q_start)
    desc = _indexer_in(q, w, keys, k_scale, path, q_scale)
    ws, nb = _workspace(ix_workspace_bytes(prob, IX_OP_INDEXER_TOPK, desc), q.device, stream)
    _check(lib.ix_indexer_topk(ctypes.byref(prob), ctypes.byref(desc), _ptr(idx), _ptr(ws), nb,
                               _stream(stream)), "ix_indexer_topk")


def ix_indexer_argmax(q, w, keys, pos, score=None, *, k_scale=None, q_start=None, kv_len=None,
                      seq_q_start=None, q_scale=None, stream=None):
    """Top-1 of the indexer scores (see ix.h): ``pos`` int32 [B, n_q] gets each
    row's best position, ``score`` (fp32 [B, n_q], optional) its score."""
    lib = load()
    _dev(pos, "pos")
    _need(pos.dtype == torch.int32 and tuple(pos.shape) == tuple(q.shape[:2]), "pos must be int32 [B, n_q]")
    if score is not None:
        _dev(score, "score")
        _need(score.dtype == torch.float32 and tuple(score.shape) == tuple(q.shape[:2]),
              "score must be fp32 [B, n_q]")
    cap = keys.shape[1]
    q_start = _starts(seq_q_start, q_start, q.shape[0])
    prob = _problem(q.shape[0], q.shape[1], q_start, cap if kv_len is None else kv_len, cap, 1, seq_q_start)
    desc = _indexer_in(q, w, keys, k_scale, IX_PATH_AUTO, q_scale)
    ws, nb = _workspace(ix_workspace_bytes(prob, IX_OP_INDEXER_ARGMAX, desc), q.device, stream)
    _check(lib.ix_indexer_argmax(ctypes.byref(prob), ctypes.byref(desc), _ptr(pos), _ptr(score), _ptr(ws), nb,
                                 _stream(stream)), "ix_indexer_argmax")


def ix_sparse_attn(q, kv, idx, out, *, lse=None, q_start=0, kv_len=None, sm_scale=0.0, kv_splits=0,
                   stream=None):
    """Sparse attention of one layer over ``idx`` into ``out`` (see ix.h)."""
    lib = load()
    _dev(idx, "idx")
    _need(idx.dtype == torch.int32 and tuple(idx.shape[:2]) == tuple(q.shape[:2]), "idx must be int32 [B, n_q, k]")
    cap = kv.shape[1]
    prob = _problem(q.shape[0], q.shape[1], q_start, cap if kv_len is None else kv_len, cap, idx.shape[2])
    desc = _attn_in(q, kv, out, lse, sm_scale, kv_splits)
    ws, nb = _workspace(ix_workspace_bytes(prob, IX_OP_SPARSE_ATTN, desc), q.device, stream)
    _check(lib.ix_sparse_attn(ctypes.byref(prob), ctypes.byref(desc), _ptr(idx), _ptr(ws), nb,
                              _stream(stream)), "ix_sparse_attn")


def _group_args(indexer_layers, attn_layers, f_mask, idx, q_start, kv_len, sm_scale, kv_splits, path,
                seq_q_start):
    n = len(attn_layers)
    _need(len(indexer_layers) == n, "one indexer entry per layer (None for shared layers)")
    _dev(idx, "idx")
    _need(idx.dtype == torch.int32 and idx.dim() == 4, "idx must be int32 [n_full, B, n_q, k]")
    a0 = attn_layers[0]
    B, n_q = a0["q"].shape[0], a0["q"].shape[1]
    cap = a0["kv"].shape[1]
    q_start = _starts(seq_q_start, q_start, B)
    prob = _problem(B, n_q, q_start, cap if kv_len is None else kv_len, cap, idx.shape[3], seq_q_start)
    ixr = (IndexerIn * n)()
    att = (AttnIn * n)()
    for l in range(n):
        if (f_mask >> l) & 1:
            e = indexer_layers[l]
            _need(e is not None, f"layer {l} is full but has no indexer inputs")
            _need(e["keys"].shape[1] == cap, "indexer keys and latent KV need the same capacity")
            ixr[l] = _indexer_in(e["q"], e["w"], e["keys"], e.get("k_scale"), path, e.get("q_scale"))
        a = attn_layers[l]
        _need(a["q"].shape[:2] == a0["q"].shape[:2] and a["kv"].shape[1] == cap, "layers must share sizes")
        att[l] = _attn_in(a["q"], a["kv"], a["out"], a.get("lse"), sm_scale, kv_splits)
    return n, prob, ixr, att, a0["q"].device


def ix_group_forward(indexer_layers, attn_layers, f_mask: int, idx, *, q_start=None, kv_len=None,
                     sm_scale=0.0, kv_splits=0, path=IX_PATH_AUTO, seq_q_start=None, stream=None):
    """One IndexShare layer group (see ix.h).

    indexer_layers[l]: dict(q=, w=, keys=, k_scale=[, q_scale=]) for full layers (None for
    shared ones); attn_layers[l]: dict(q=, kv=, out=, lse=).  Bit l of f_mask
    marks layer l full.  idx: int32 [n_full, B, n_q, k].  ``seq_q_start`` as
    in ix_indexer_topk."""
    lib = load()
    n, prob, ixr, att, dev = _group_args(indexer_layers, attn_layers, f_mask, idx, q_start, kv_len, sm_scale,
                                         kv_splits, path, seq_q_start)
    gd = GroupDesc(n, 0, f_mask, ixr, att)
    ws, nb = _workspace(ix_workspace_bytes(prob, IX_OP_GROUP_FORWARD, gd), dev, stream)
    _check(lib.ix_group_forward(ctypes.byref(prob), n, f_mask, ixr, att, _ptr(idx), _ptr(ws), nb,
                                _stream(stream)), "ix_group_forward")


def ix_group_forward_noalloc(indexer_layers, attn_layers, f_mask: int, idx, *, q_start=None, kv_len=None,
                             sm_scale=0.0, kv_splits=0, path=IX_PATH_AUTO, seq_q_start=None, stream=None):
    """ix_group_forward in the library's static scratch: no workspace is
    allocated, by this binding or the library (see ix.h; calls that overlap
    on one GPU race on the scratch)."""
    lib = load()
    n, prob, ixr, att, _ = _group_args(indexer_layers, attn_layers, f_mask, idx, q_start, kv_len, sm_scale,
                                       kv_splits, path, seq_q_start)
    _check(lib.ix_group_forward_noalloc(ctypes.byref(prob), n, f_mask, ixr, att, _ptr(idx), _stream(stream)),
           "ix_group_forward_noalloc")


def ix_topk_scores(scores, idx, *, q_start=None, kv_len=None, seq_q_start=None, stream=None):
    """Top-k over fp32 score rows ``scores`` [B, n_q, ld] into idx [B, n_q, k]
    (``seq_q_start`` as in ix_indexer_topk)."""
    lib = load()
    _dev(scores, "scores"), _dev(idx, "idx")
    _need(scores.dtype == torch.float32 and scores.dim() == 3, "scores must be fp32 [B, n_q, ld]")
    _need(idx.dtype == torch.int32 and tuple(idx.shape[:2]) == tuple(scores.shape[:2]), "idx must be int32 [B, n_q, k]")
    ld = scores.shape[2]
    q_start = _starts(seq_q_start, q_start, scores.shape[0])
    prob = _problem(scores.shape[0], scores.shape[1], q_start, ld if kv_len is None else kv_len,
                    ld if kv_len is None else kv_len, idx.shape[2], seq_q_start)
    ws, nb = _workspace(ix_workspace_bytes(prob, IX_OP_TOPK_SCORES, None), scores.device, stream)
    _check(lib.ix_topk_scores(ctypes.byref(prob), _ptr(scores), ld, _ptr(idx), _ptr(ws), nb,
                              _stream(stream)), "ix_topk_scores")


def ix_index_overlap(idx_a, idx_b, counts=None, *, stream=None):
    """Per-row count of positions present in both index buffers [B, n_q, k]
    (negative slots ignored) into ``counts`` int32 [B, n_q] (see ix.h)."""
    lib = load()
    _dev(idx_a, "idx_a"), _dev(idx_b, "idx_b")
    _need(idx_a.dtype == torch.int32 and idx_a.dim() == 3 and idx_b.shape == idx_a.shape
          and idx_b.dtype == torch.int32, "idx_a, idx_b must be int32 [B, n_q, k] of one shape")
    B, n_q, k = idx_a.shape
    if counts is None:
        counts = torch.empty((B, n_q), dtype=torch.int32, device=idx_a.device)
    _dev(counts, "counts")
    _need(counts.dtype == torch.int32 and tuple(counts.shape) == (B, n_q), "counts must be int32 [B, n_q]")
    prob = _problem(B, n_q, 0, n_q, n_q, k)
    _check(lib.ix_index_overlap(ctypes.byref(prob), _ptr(idx_a), _ptr(idx_b), _ptr(counts),
                                _stream(stream)), "ix_index_overlap")
    return counts


def ix_append_keys(k_new, k_cache, k_scale, pos=None, *, seq_pos=None, stream=None):
    """Quantize new fp32 key rows ``k_new`` [B, n_new, d] into the fp8 key
    cache ``k_cache`` (uint8 e4m3fn codes [B, kv_cap, d]) and ``k_scale``
    (fp32 [B, kv_cap]) at rows [pos, pos + n_new) (see ix.h).

    ``seq_pos`` (int64 [B] on the device, optional): each sequence's own first
    row instead; ``pos`` is then their bound (default: their maximum)."""
    lib = load()
    _dev(k_new, "k_new"), _dev(k_cache, "k_cache"), _dev(k_scale, "k_scale")
    _need(k_new.dtype == torch.float32 and k_new.dim() == 3, "k_new must be fp32 [B, n_new, d]")
    kc = k_cache.view(torch.uint8) if k_cache.dtype == torch.float8_e4m3fn else k_cache
    _need(kc.dtype == torch.uint8 and kc.dim() == 3 and kc.shape[0] == k_new.shape[0]
          and kc.shape[2] == k_new.shape[2], "k_cache must be e4m3fn codes [B, kv_cap, d]")
    _need(k_scale.dtype == torch.float32 and tuple(k_scale.shape) == tuple(kc.shape[:2]),
          "k_scale must be fp32 [B, kv_cap]")
    B, n_new, d = k_new.shape
    cap = kc.shape[1]
    _need(pos is not None or seq_pos is not None, "give pos or seq_pos")
    pos = _starts(seq_pos, pos, B)
    # with per-sequence rows the bound pos is the problem's q_start, so row
    # pos_b = pos - q_start + seq_pos[b] = seq_pos[b]
    prob = _problem(B, 1, 0 if seq_pos is None else pos, cap, cap, 1, seq_pos)
    _check(lib.ix_append_keys(ctypes.byref(prob), d, _ptr(k_new), n_new, int(pos), _ptr(kc), _ptr(k_scale),
                              _stream(stream)), "ix_append_keys")


def ix_indexer_project(x, w_proj, q_out, w_out, *, heads, dim, stream=None):
    """Indexer queries and head weights from hidden states (see ix.h):
    ``x`` bf16 [..., d_in] (rows flattened), ``w_proj`` bf16
    [heads*dim + heads, d_in] -> ``q_out`` bf16 [..., heads, dim] (rounded to
    nearest, ties to even) and ``w_out`` fp32 [..., heads]."""
    lib = load()
    for t, name in ((x, "x"), (w_proj, "w_proj"), (q_out, "q_out"), (w_out, "w_out")):
        _dev(t, name)
    _need(x.dtype == torch.bfloat16 and x.dim() >= 1, "x must be bf16 [..., d_in]")
    d_in = x.shape[-1]
    rows = x.numel() // d_in if d_in else 0
    _need(w_proj.dtype == torch.bfloat16 and tuple(w_proj.shape) == (heads * dim + heads, d_in),
          "w_proj must be bf16 [heads*dim + heads, d_in]")
    _need(q_out.dtype == torch.bfloat16 and tuple(q_out.shape) == tuple(x.shape[:-1]) + (heads, dim),
          "q_out must be bf16 [..., heads, dim]")
    _need(w_out.dtype == torch.float32 and tuple(w_out.shape) == tuple(x.shape[:-1]) + (heads,),
          "w_out must be fp32 [..., heads]")
    if rows == 0:
        return                                   # nothing to do (empty tensors may hold no pointer)
    pin = ProjectIn(heads, dim, d_in, 0, _ptr(x), _ptr(w_proj))
    _check(lib.ix_indexer_project(rows, ctypes.byref(pin), _ptr(q_out), _ptr(w_out), _stream(stream)),
           "ix_indexer_project")


def ix_quantize_queries(q, codes=None, scale=None, *, stream=None):
    """bf16 indexer queries [..., d] -> (e4m3fn codes uint8 [..., d], fp32
    scale [...]), one scale per row of d values (see ix.h): the ``q`` and
    ``q_scale`` of the fp8-query indexer.  Returns (codes, scale)."""
    lib = load()
    _dev(q, "q")
    _need(q.dtype == torch.bfloat16 and q.dim() >= 1 and q.is_contiguous(), "q must be contiguous bf16 [..., d]")
    d = q.shape[-1]
    if codes is None:
        codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _dev(codes, "codes"), _dev(scale, "scale")
    _need(codes.dtype == torch.uint8 and tuple(codes.shape) == tuple(q.shape) and codes.is_contiguous(),
          "codes must be contiguous uint8 of q's shape")
    _need(scale.dtype == torch.float32 and tuple(scale.shape) == tuple(q.shape[:-1]) and scale.is_contiguous(),
          "scale must be contiguous fp32 of q's shape without its last dim")
    n_rows = q.numel() // d if d else 0
    if n_rows == 0:
        return codes, scale
    _check(lib.ix_quantize_queries(n_rows, d, _ptr(q), _ptr(codes), _ptr(scale), _stream(stream)),
           "ix_quantize_queries")
    return codes, scale
