"""CPU oracle for the DSA layer group under the IndexShare schedule.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares no code with the GPU library: it reads raw input bytes
(bf16 bit patterns, e4m3fn codes, fp32) and computes everything in float64
with plain NumPy, following the definitions on the pages:

* "IndexShare" (LLM Architecture Gallery), section "Why The Indexer Becomes
  Expensive": a lightweight indexer scores the preceding tokens of a query and
  keeps the top-k positions; the main attention then runs on that subset only.
* "GLM-5.2 and IndexShare for Long-Context Sparse Attention", section "Where
  the DSA indexer becomes expensive": the indexer keeps the top 2,048 earlier
  tokens for each query position.
* "IndexShare" (LLM Architecture Gallery), section "How IndexShare Works": a
  full layer runs the indexer, does the top-k and stores the selected
  positions; a shared layer skips both and reuses the most recent full layer's
  positions; only the integer positions cross layers.
* "IndexCache: Killing the Indexer's O(NL^2) Bottleneck" notes, section 2:
  F layers compute fresh top-k, S layers reuse the nearest preceding F layer's
  result, and the first layer is always F.

Readings taken where the pages are silent:
* indexer score: score(t, s) = sum_h w[t, h] * max(0, q[t, h, :] . k[s, :]),
  one key vector per token shared by all indexer heads (the pages describe
  the indexer only as a small, low-rank module with few heads, in FP8);
* a query at absolute position p may select any s with 0 <= s <= p (itself
  included), and s < kv_len;
* order: larger score first, equal scores -> lower position first; the row is
  emitted as ascending positions, padded with -1 to length k;
* fp8 keys are e4m3fn codes times a per-row fp32 scale; queries may be given
  the same way, as e4m3fn codes times one fp32 scale per (row, head) (the
  pages' FP8 indexer taken as an input format, a mode declared by the caller;
  the default queries are bf16);
* attention over the selected rows: o = softmax(sm_scale * Q K^T) V with K the
  whole latent row and V its first d_v dims; slots holding -1 (or any value
  outside [0, kv_len)) are ignored; a row with no valid slot gives o = 0 and
  lse = -inf;
* sequences of different lengths in one batch: row t of sequence b sits at
  its own start q_start[b] + t, with the same candidate rule;
* MTP draft steps after the first attend over the first step's positions in
  the first step's KV cache, so no position a later step adds is selected;
* the indexer's inputs from hidden states (IndexCache notes, section 1: a
  small low-rank indexer with few heads): one bf16 input row x per query and
  one bf16 weight W of H*d + H rows give [q_I | w] = x . W^T; q_I is rounded
  to bf16 (nearest, ties to the even pattern), the head weights stay wide.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3fn", "key_matrix", "indexer_scores", "select_topk",
    "indexer_topk", "indexer_topk_rows", "attention_row", "sparse_attention", "group_forward",
    "mtp_draft", "index_overlap", "encode_e4m3fn", "quantize_key_rows", "encode_bf16",
    "indexer_project", "query_matrix",
]


# ---------------------------------------------------------------- decoding --
def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the upper half
    of an IEEE binary32 word, so widening is a 16-bit shift."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """OCP FP8 E4M3FN codes (uint8) -> float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds subnormals m * 2^-9; code 0x7F/0xFF is NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)
    return sign * v


def key_matrix(keys, key_dtype: str, scale=None) -> np.ndarray:
    """Stored indexer keys [..., n, d] -> float64 values (codes times the row
    scale for fp8)."""
    if key_dtype == "bf16":
        return decode_bf16(keys)
    if key_dtype == "fp8":
        v = decode_e4m3fn(keys)
        return v * np.asarray(scale, dtype=np.float64)[..., None]
    raise ValueError(f"unknown key dtype {key_dtype!r}")


def query_matrix(q, q_scale=None) -> np.ndarray:
    """Indexer queries [..., H, d] -> float64 values: bf16 bit patterns, or,
    with q_scale [..., H], e4m3fn codes times their (row, head) scale."""
    if q_scale is None:
        return decode_bf16(q)
    return decode_e4m3fn(q) * np.asarray(q_scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------- key quantizing --
E4M3FN_MAX = 448.0


def encode_e4m3fn(x) -> np.ndarray:
    """float values -> OCP FP8 E4M3FN codes (uint8), round to nearest with ties
    to the code whose last bit is 0, saturating at +-448 (no NaN input).

    Written as a plain nearest-value search over the 253 finite codes'
    decoded values, not as bit arithmetic."""
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    finite = ~np.isnan(vals) & ~((codes == 0x80))          # keep one zero (+0)
    cand_codes = codes[finite]
    cand_vals = vals[finite]
    a = np.clip(np.asarray(x, dtype=np.float64), -E4M3FN_MAX, E4M3FN_MAX)
    flat = a.reshape(-1)
    out = np.empty(flat.shape[0], dtype=np.uint8)
    for i, v in enumerate(flat):
        d = np.abs(cand_vals - v)
        best = np.flatnonzero(d == d.min())
        if best.shape[0] > 1:                               # a tie: the even code
            best = best[(cand_codes[best] & 1) == 0]
        c = cand_codes[best[0]]
        if c == 0 and v < 0:                                # a negative value rounding to zero keeps its sign
            c = np.uint8(0x80)
        out[i] = c
    return out.reshape(a.shape)


def quantize_key_rows(k_rows):
    """New indexer key rows (fp32 [..., d]) -> (e4m3fn codes [..., d], fp32
    scales [...]) in the cache format.

    IndexCache notes, section 1: the indexer keys are stored in FP8.  Reading
    of the per-row scaling (the pages give none): scale = max_j |k_j| / 448,
    or 1 for an all-zero row, and code_j = e4m3fn(k_j / scale); the scale and
    the division are single-precision operations, as the stored format is."""
    k = np.asarray(k_rows, dtype=np.float32)
    amax = np.abs(k).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3FN_MAX), np.float32(1.0)).astype(np.float32)
    y = (k / scale[..., None]).astype(np.float32)
    return encode_e4m3fn(y), scale


# ---------------------------------------------------------- indexer inputs --
def encode_bf16(x) -> np.ndarray:
    """finite float values -> bf16 bit patterns (uint16), round to nearest with
    ties to the pattern whose last bit is 0.

    bf16 keeps 8 significant bits.  A nonzero v = f * 2^e with 0.5 <= |f| < 1
    is rounded as an integer multiple of 2^(e - 8) (a power-of-two scaling,
    exact in float64); np.rint rounds halves to even, and an even multiple is
    a pattern with last bit 0.  The rounded value is a bf16 value, so its
    float32 image carries the pattern in its upper 16 bits.  (Values below
    the normal range do not occur in this library's uses.)"""
    v = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(v)
    step = np.ldexp(1.0, e - 8)
    r = np.where(v == 0.0, v, np.rint(v / step) * step)
    bits = r.astype(np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def indexer_project(x_bits, w_bits, heads: int, dim: int):
    """Indexer queries and head weights from hidden-state rows.

    x_bits: bf16 patterns [rows, d_in]; w_bits: bf16 patterns [heads*dim +
    heads, d_in] (one row per output column).  y = x . W^T in float64; the
    first heads*dim columns, rounded to bf16, are q_I [rows, heads, dim]
    (uint16 patterns); the last heads columns are w [rows, heads] (float64).
    IndexCache notes, section 1 (a small low-rank indexer with few heads);
    the shapes and the single input are this library's reading."""
    X = decode_bf16(x_bits)
    W = decode_bf16(w_bits)
    if W.shape[0] != heads * dim + heads or W.shape[1] != X.shape[-1]:
        raise ValueError("w must be [heads*dim + heads, d_in]")
    Y = X @ W.T
    q = encode_bf16(Y[..., : heads * dim]).reshape(X.shape[:-1] + (heads, dim))
    return q, Y[..., heads * dim:]


# ----------------------------------------------------------------- indexer --
def indexer_scores(q_row: np.ndarray, w_row: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """score[s] = sum_h w[h] * max(0, q[h, :] . keys[s, :]) in float64.

    q_row [H, d], w_row [H], keys [n, d] (already decoded) -> [n].
    """
    x = keys @ q_row.T                       # [n, H]: one dot product per head
    return np.maximum(x, 0.0) @ w_row        # weighted sum of the ReLU'd heads


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The first min(k, n) positions under (score desc, position asc),
    returned in ascending position order and padded with -1 to length k.

    A stable sort of -score keeps ascending position among equal scores
    (+0.0 and -0.0 compare equal)."""
    n = scores.shape[0]
    order = np.argsort(-scores, kind="stable")
    sel = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


def indexer_topk(q, w, keys, key_dtype, scale, q_start, kv_len: int, k: int,
                 rows=None, q_scale=None) -> np.ndarray:
    """Full-layer indexer + top-k for every (sequence, query row).

    q: bf16 bits [B, n_q, H, d]; w: fp32 [B, n_q, H]; keys: [B, cap, d] bf16
    bits or e4m3fn codes; scale: [B, cap] fp32 (fp8 only).  q_start: the
    position of query row 0, one int for every sequence or one per sequence
    (a batch of sequences of different lengths: row t of sequence b sits at
    q_start[b] + t and may select the keys up to there, as any query does).
    ``rows`` limits the work to the listed query rows (the result then has
    len(rows) rows).  With q_scale [B, n_q, H], q holds e4m3fn codes (see
    query_matrix).  Returns int32 [B, len(rows), k].
    """
    q = np.asarray(q)
    B, n_q = q.shape[0], q.shape[1]
    starts = ([int(q_start)] * B if np.ndim(q_start) == 0
              else [int(x) for x in np.asarray(q_start).reshape(-1)])
    if len(starts) != B:
        raise ValueError("q_start needs one entry per sequence")
    rows = list(range(n_q)) if rows is None else list(rows)
    out = np.full((B, len(rows), k), -1, dtype=np.int32)
    for b in range(B):
        p_max = min(starts[b] + max(rows), kv_len - 1)
        sc = None if scale is None else np.asarray(scale)[b, : p_max + 1]
        kmat = key_matrix(np.asarray(keys)[b, : p_max + 1], key_dtype, sc)
        for i, t in enumerate(rows):
            p = starts[b] + t
            n = min(p, kv_len - 1) + 1
            qs = None if q_scale is None else np.asarray(q_scale)[b, t]
            s = indexer_scores(query_matrix(q[b, t], qs), np.asarray(w[b, t], np.float64),
                               kmat[:n])
            out[b, i] = select_topk(s, k)
    return out


def indexer_topk_rows(q_rows, w_rows, keys_b, key_dtype, scale_b, positions, kv_len: int,
                      k: int, q_scale_rows=None) -> np.ndarray:
    """Indexer + top-k for individual query rows of one sequence, given their
    absolute positions (decodes the reachable keys once).

    q_rows: bf16 bits [R, H, d]; w_rows: fp32 [R, H]; keys_b: [cap, d] of one
    sequence; scale_b: [cap] (fp8 only); positions: [R]; q_scale_rows: [R, H]
    for e4m3fn-coded queries.  Returns int32 [R, k].
    """
    positions = [int(p) for p in positions]
    p_max = min(max(positions), kv_len - 1)
    sc = None if scale_b is None else np.asarray(scale_b)[: p_max + 1]
    kmat = key_matrix(np.asarray(keys_b)[: p_max + 1], key_dtype, sc)
    out = np.full((len(positions), k), -1, dtype=np.int32)
    for i, p in enumerate(positions):
        n = min(p, kv_len - 1) + 1
        qs = None if q_scale_rows is None else np.asarray(q_scale_rows)[i]
        s = indexer_scores(query_matrix(q_rows[i], qs), np.asarray(w_rows[i], np.float64), kmat[:n])
        out[i] = select_topk(s, k)
    return out


# --------------------------------------------------------------- attention --
def attention_row(q_row: np.ndarray, kv: np.ndarray, sel: np.ndarray, sm_scale: float,
                  d_v: int):
    """Exact softmax attention of one query row over the latent rows ``sel``.

    q_row [Hq, D] float64; kv [n, D] float64 (all rows); sel: valid row ids.
    Returns (o [Hq, d_v], lse [Hq]) in float64.
    """
    hq = q_row.shape[0]
    if sel.size == 0:
        return np.zeros((hq, d_v)), np.full(hq, -np.inf)
    rows = kv[sel]                                   # [m, D]
    z = sm_scale * (q_row @ rows.T)                  # [Hq, m]
    mx = z.max(axis=1, keepdims=True)
    p = np.exp(z - mx)
    den = p.sum(axis=1)
    o = (p @ rows[:, :d_v]) / den[:, None]
    return o, mx[:, 0] + np.log(den)


def sparse_attention(Q, KV, idx, kv_len: int, sm_scale: float, d_v: int, rows=None,
                     idx_rows=None):
    """Sparse attention of every query row over its selected positions.

    Q: bf16 bits [B, n_q, Hq, D]; KV: bf16 bits [B, cap, D]; idx: int32
    [B, n_idx, k].  ``rows`` picks the query rows; ``idx_rows`` gives, for each
    of them, its row in ``idx`` (default: the same index).  Slots outside
    [0, kv_len) are ignored.  Returns (O [B, R, Hq, d_v], lse [B, R, Hq]).
    """
    Q = np.asarray(Q)
    B, n_q, hq, _ = Q.shape
    rows = list(range(n_q)) if rows is None else list(rows)
    idx_rows = rows if idx_rows is None else list(idx_rows)
    O = np.zeros((B, len(rows), hq, d_v))
    L = np.zeros((B, len(rows), hq))
    for b in range(B):
        for i, (t, it) in enumerate(zip(rows, idx_rows)):
            r = np.asarray(idx[b, it]).astype(np.int64)
            sel = r[(r >= 0) & (r < kv_len)]
            kv = decode_bf16(np.asarray(KV)[b, sel])    # decode only the rows used
            O[b, i], L[b, i] = attention_row(decode_bf16(Q[b, t]), kv,
                                             np.arange(sel.size), sm_scale, d_v)
    return O, L


# ---------------------------------------------------------------- schedule --
def group_forward(roles: str, indexer_layers, attn_layers, q_start, kv_len: int,
                  k: int, sm_scale: float, d_v: int, rows=None):
    """Walk one IndexShare layer group.

    roles: one letter per layer, "F" (runs indexer + top-k and stores the
    positions) or "S" (reuses the most recent F layer's positions untouched).
    indexer_layers[l] = (q, w, keys, key_dtype, scale[, q_scale]) — read for
    F layers only; attn_layers[l] = (Q, KV).  q_start as in indexer_topk (one int, or
    one per sequence).  Returns a dict with per-layer outputs
    "O"/"lse", the list "idx" of index buffers (one per F layer), "used" (for
    each layer, which F buffer it attended over) and "n_indexer_runs".
    """
    if not roles or roles[0] != "F":
        raise ValueError("the first layer of a group must be a full (F) layer")
    cur = None
    idx_list, used, outs, lses = [], [], [], []
    runs = 0
    for l, role in enumerate(roles):
        if role == "F":
            q, w, keys, kd, sc, *qsc = indexer_layers[l]
            cur = indexer_topk(q, w, keys, kd, sc, q_start, kv_len, k, rows=rows,
                               q_scale=qsc[0] if qsc else None)
            idx_list.append(cur)
            runs += 1
        elif role != "S":
            raise ValueError(f"unknown role {role!r}")
        used.append(len(idx_list) - 1)
        Q, KV = attn_layers[l]
        n_r = cur.shape[1]
        o, lse = sparse_attention(Q, KV, cur, kv_len, sm_scale, d_v, rows=rows,
                                  idx_rows=range(n_r))
        outs.append(o)
        lses.append(lse)
    return {"O": outs, "lse": lses, "idx": idx_list, "used": used, "n_indexer_runs": runs}


def mtp_draft(indexer_in, draft_q, kv, q_start, kv_len: int, k: int, sm_scale: float, d_v: int,
              rows=None):
    """Draft steps of the multi-token-prediction (MTP) layer with index reuse.

    "GLM-5.2 and IndexShare for Long-Context Sparse Attention", section "Reuse
    in the MTP layer": the first draft step runs the indexer and keeps its
    positions; every later draft step attends over those same positions in
    the same, earlier KV cache (nothing the later steps add is selected).
    indexer_in = (q, w, keys, key_dtype, scale[, q_scale]) of the first step's query rows
    (positions q_start + t); draft_q: one bf16-bit Q [B, n_q, Hq, D] per draft
    step; kv: the MTP layer's latent cache [B, cap, D], shared by all steps.
    Returns dict(idx, O: list per step, lse: list per step, n_indexer_runs).
    """
    if len(draft_q) < 1:
        raise ValueError("at least one draft step")
    q, w, keys, kd, sc, *qsc = indexer_in
    idx = indexer_topk(q, w, keys, kd, sc, q_start, kv_len, k, rows=rows,
                       q_scale=qsc[0] if qsc else None)
    outs, lses = [], []
    for Q in draft_q:
        o, lse = sparse_attention(Q, kv, idx, kv_len, sm_scale, d_v, rows=rows,
                                  idx_rows=range(idx.shape[1]))
        outs.append(o)
        lses.append(lse)
    return {"idx": idx, "O": outs, "lse": lses, "n_indexer_runs": 1}


# ------------------------------------------------------------- diagnostics --
def index_overlap(idx_a, idx_b) -> np.ndarray:
    """Per row, the number of positions selected in both index rows.

    "IndexShare" (LLM Architecture Gallery), section "Why Reusing Indices Can
    Work": reuse pays off because the top-k sets of adjacent layers overlap
    heavily; this is that count, |{valid a} & {valid b}| for each row, with
    negative slots (the -1 padding) ignored.  idx_a, idx_b: integer arrays of
    the same shape [..., k]; returns int64 [...].
    """
    a = np.asarray(idx_a)
    b = np.asarray(idx_b)
    if a.shape != b.shape:
        raise ValueError("index buffers must have the same shape")
    lead = a.shape[:-1]
    a2 = a.reshape(-1, a.shape[-1])
    b2 = b.reshape(-1, b.shape[-1])
    out = np.empty(a2.shape[0], dtype=np.int64)
    for r in range(a2.shape[0]):
        sa = set(int(x) for x in a2[r] if x >= 0)
        sb = set(int(x) for x in b2[r] if x >= 0)
        out[r] = len(sa & sb)
    return out.reshape(lead)

