"""Plant plausible mistakes in the CPU oracle and check that the pins catch
each one (the pins are only worth something if they fail on a wrong oracle).
CPU only; every mutation is undone by monkeypatch."""
import numpy as np
import pytest

from oracle import dsa_oracle as O
import test_oracle_pins as P


def _no_relu(q_row, w_row, keys):
    return (keys @ q_row.T) @ w_row


def _abs_weights(q_row, w_row, keys):
    return np.maximum(keys @ q_row.T, 0.0) @ np.abs(w_row)


def _transposed_q(q_row, w_row, keys):
    # the hand-worked example is square (H = d = 2), so q^T has q's shape
    return np.maximum(keys @ q_row, 0.0) @ w_row


def _ties_to_higher_position(scores, k):
    n = scores.shape[0]
    order = np.lexsort((-np.arange(n), -scores))       # equal scores: higher position first
    sel = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


def _score_order_output(scores, k):
    n = scores.shape[0]
    order = np.argsort(-scores, kind="stable")[: min(k, n)]
    out = np.full(k, -1, dtype=np.int32)
    out[: order.shape[0]] = order
    return out


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    v = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    v = np.where((e == 0xF) & ((c & 7) == 7), np.nan, v)
    return sign * v


def _attn_wrong_v(q_row, kv, sel, sm_scale, d_v):
    rows = kv[sel]
    z = sm_scale * (q_row @ rows.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    den = p.sum(axis=1)
    return (p @ rows[:, -d_v:]) / den[:, None], z.max(axis=1) + np.log(den)


def _attn_no_scale(q_row, kv, sel, sm_scale, d_v):
    return ATTN(q_row, kv, sel, 1.0, d_v)


def _overlap_counts_padding(idx_a, idx_b):
    a, b = np.asarray(idx_a), np.asarray(idx_b)
    return np.array([len(set(x.tolist()) & set(y.tolist())) for x, y in
                     zip(a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1]))]).reshape(a.shape[:-1])


def _overlap_slotwise(idx_a, idx_b):
    a, b = np.asarray(idx_a), np.asarray(idx_b)
    return ((a == b) & (a >= 0)).sum(axis=-1)


def _encode_ties_away(x):
    codes = np.arange(256, dtype=np.uint8)
    vals = O.decode_e4m3fn(codes)
    keep = ~np.isnan(vals)
    cv, cc = vals[keep], codes[keep]
    a = np.clip(np.asarray(x, dtype=np.float64), -448.0, 448.0).reshape(-1)
    out = np.empty(a.shape[0], dtype=np.uint8)
    for i, v in enumerate(a):
        d = np.abs(cv - v)
        best = np.flatnonzero(d == d.min())
        out[i] = cc[best[np.argmax(np.abs(cv[best]))]]      # ties away from zero
    return out.reshape(np.shape(x))


def _quantize_fnuz_max(k_rows):
    k = np.asarray(k_rows, dtype=np.float32)
    amax = np.abs(k).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(240.0), np.float32(1.0)).astype(np.float32)
    return O.encode_e4m3fn((k / scale[..., None]).astype(np.float32)), scale


def _bf16_truncate(x):
    v = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _project_weights_first(x_bits, w_bits, heads, dim):
    X, W = O.decode_bf16(x_bits), O.decode_bf16(w_bits)
    Y = X @ W.T
    q = O.encode_bf16(Y[..., heads:]).reshape(X.shape[:-1] + (heads, dim))
    return q, Y[..., :heads]


def _query_scale_ignored(q, q_scale=None):
    return O.decode_bf16(q) if q_scale is None else O.decode_e4m3fn(q)


ATTN = O.attention_row
INDEXER = O.indexer_topk

HAND = {c["p"] * 100 + c["k"]: c for c in P.gold()["indexer"]["cases"]}

MUTATIONS = [
    ("drop_relu", "indexer_scores", _no_relu, lambda: P.test_hand_worked_indexer_topk(HAND[403])),
    ("abs_weights", "indexer_scores", _abs_weights, lambda: P.test_hand_worked_indexer_topk(HAND[402])),
    ("transposed_q", "indexer_scores", _transposed_q, P.test_hand_worked_indexer_scores),
    ("ties_high_pos", "select_topk", _ties_to_higher_position, P.test_select_topk_brute_force_tiny),
    ("score_order", "select_topk", _score_order_output, lambda: P.test_hand_worked_indexer_topk(HAND[402])),
    ("e4m3_bias", "decode_e4m3fn", _e4m3_bias8, P.test_e4m3fn_decode_matches_torch_for_all_256_codes),
    ("wrong_v_slice", "attention_row", _attn_wrong_v, P.test_hand_worked_attention),
    ("no_sm_scale", "attention_row", _attn_no_scale, P.test_attention_with_full_prefix_equals_dense_causal_sdpa),
    ("overlap_counts_padding", "index_overlap", _overlap_counts_padding,
     P.test_overlap_ignores_padding_and_is_symmetric),
    ("overlap_slotwise", "index_overlap", _overlap_slotwise, P.test_overlap_shifted_ranges_closed_form),
    ("e4m3_ties_away", "encode_e4m3fn", _encode_ties_away, P.test_e4m3fn_encode_matches_torch_on_grid_and_midpoints),
    ("quantize_fnuz_range", "quantize_key_rows", _quantize_fnuz_max, P.test_quantize_rows_closed_forms),
    ("bf16_truncate", "encode_bf16", _bf16_truncate, P.test_projection_rounds_midpoints_to_even),
    ("project_weights_first", "indexer_project", _project_weights_first, P.test_hand_worked_projection),
    ("query_scale_ignored", "query_matrix", _query_scale_ignored, P.test_hand_worked_fp8_queries),
]


@pytest.mark.parametrize("name,attr,fn,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, name, attr, fn, check):
    check()                                   # passes on the real oracle
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        check()


def test_pins_catch_varlen_sharing_one_start(monkeypatch):
    """Giving every sequence the largest start (the per-sequence starts
    ignored) fails the brute-force batch pin."""
    def one_start(q, w, keys, key_dtype, scale, q_start, kv_len, k, rows=None):
        return INDEXER(q, w, keys, key_dtype, scale, int(np.max(q_start)), kv_len, k, rows)
    P.test_varlen_batch_brute_force_tiny()
    monkeypatch.setattr(O, "indexer_topk", one_start)
    with pytest.raises(AssertionError):
        P.test_varlen_batch_brute_force_tiny()


def test_pins_catch_mtp_steps_selecting_again(monkeypatch):
    """Later draft steps that rerun the selection at their own positions (and
    so see the rows the cache holds past the first step) fail the MTP pin."""
    def reselect(indexer_in, draft_q, kv, q_start, kv_len, k, sm_scale, d_v, rows=None):
        q, w, keys, kd, sc = indexer_in
        outs, lses = [], []
        for j, Q in enumerate(draft_q):
            idx = INDEXER(q, w, keys, kd, sc, q_start + j, kv_len, k, rows=rows)
            o, lse = O.sparse_attention(Q, kv, idx, kv_len, sm_scale, d_v, rows=rows,
                                        idx_rows=range(idx.shape[1]))
            outs.append(o)
            lses.append(lse)
        return {"idx": idx, "O": outs, "lse": lses, "n_indexer_runs": 1}
    P.test_mtp_draft_later_steps_attend_over_the_first_steps_prefix()
    monkeypatch.setattr(O, "mtp_draft", reselect)
    with pytest.raises(AssertionError):
        P.test_mtp_draft_later_steps_attend_over_the_first_steps_prefix()


def test_pins_catch_self_excluded_causality(monkeypatch):
    """A query that may not select its own position changes the hand-worked
    p=4, k=5 row (position 4 would be missing)."""
    def excl(q, w, keys, key_dtype, scale, q_start, kv_len, k, rows=None):
        out = INDEXER(q, w, keys, key_dtype, scale, q_start, kv_len, k, rows)
        return np.where(out == q_start, -1, out)
    monkeypatch.setattr(O, "indexer_topk", excl)
    with pytest.raises(AssertionError):
        P.test_hand_worked_indexer_topk(HAND[405])
