"""Pins for the CPU oracle: checked against hand-worked examples, library
routines, brute force on tiny inputs and closed forms -- never against itself.
CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dsa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def bf16_bits(x) -> np.ndarray:
    """float values (exactly representable in bf16) -> bf16 bit patterns."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.as_tensor(np.asarray(x, dtype=np.float32))), \
        "fixture value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def gold():
    with open(GOLD) as f:
        return json.load(f)


# ------------------------------------------------------------- decoders ----
def test_e4m3fn_decode_matches_torch_for_all_256_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().double().numpy()
    got = O.decode_e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                     # 0x7F and 0xFF only: no infinities
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = O.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~ok)
    np.testing.assert_array_equal(got[ok], ref[ok])


# ----------------------------------------------------- hand-worked cases ----
def _hand_inputs(g):
    ix = g["indexer"]
    q = bf16_bits(ix["q"])[None, None]                      # [1, 1, H, d]
    w = np.asarray(ix["w"], np.float32)[None, None]
    keys = bf16_bits(ix["keys"])[None]                      # [1, 5, d]
    return q, w, keys


def test_hand_worked_indexer_scores():
    g = gold()
    q, w, keys = _hand_inputs(g)
    s = O.indexer_scores(O.decode_bf16(q[0, 0]), w[0, 0].astype(np.float64),
                         O.key_matrix(keys[0], "bf16"))
    np.testing.assert_array_equal(s, g["indexer"]["scores_p4"])


@pytest.mark.parametrize("case", gold()["indexer"]["cases"], ids=lambda c: f"p{c['p']}k{c['k']}")
def test_hand_worked_indexer_topk(case):
    q, w, keys = _hand_inputs(gold())
    idx = O.indexer_topk(q, w, keys, "bf16", None, q_start=case["p"], kv_len=5, k=case["k"])
    assert idx.tolist() == [[case["idx"]]]


def test_hand_worked_attention():
    a = gold()["attention"]
    Q = bf16_bits(a["q"])[None, None]
    KV = bf16_bits(a["kv"])[None]
    idx = np.asarray(a["idx"], np.int32)[None, None]
    o, lse = O.sparse_attention(Q, KV, idx, a["kv_len"], math.log(2.0), a["d_v"])
    np.testing.assert_allclose(o[0, 0], a["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(np.exp(lse[0, 0]), a["lse_exp"], rtol=1e-14)


# ------------------------------------------------------------- brute force --
def _brute_topk(scores, k):
    """Enumerate every subset of size min(k, n); the answer is the unique one
    in which each member beats each non-member (higher score, or equal score
    and lower position)."""
    n = len(scores)
    m = min(k, n)
    found = []
    for sub in itertools.combinations(range(n), m):
        inside = set(sub)
        if all((scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
               for i in inside for j in range(n) if j not in inside):
            found.append(sub)
    assert len(found) == 1
    return list(found[0]) + [-1] * (k - m)


def test_select_topk_brute_force_tiny():
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 10))
        scores = rng.integers(-2, 3, size=n).astype(np.float64)   # many ties
        if trial % 3 == 0:
            scores = scores * -0.0 + scores                       # keep -0.0/+0.0 mixes
            scores[scores == 0] = np.where(rng.random(np.sum(scores == 0)) < 0.5, -0.0, 0.0)
        assert O.select_topk(scores, k).tolist() == _brute_topk(list(scores), k)


def test_indexer_topk_brute_force_tiny_end_to_end():
    """Whole indexer on tiny integer inputs against scores summed by explicit
    loops and the subset-enumeration selection."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        H, d, n = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(2, 8))
        qv = rng.integers(-3, 4, size=(H, d)).astype(np.float32)
        kv = rng.integers(-3, 4, size=(n, d)).astype(np.float32)
        wv = rng.choice([-2.0, -1.0, 1.0, 2.0, 4.0], size=H).astype(np.float32)
        k = int(rng.integers(1, n + 2))
        p = n - 1
        ref = []
        for s in range(n):
            tot = 0.0
            for h in range(H):
                dot = 0.0
                for j in range(d):
                    dot += float(qv[h, j]) * float(kv[s, j])
                tot += float(wv[h]) * (dot if dot > 0 else 0.0)
            ref.append(tot)
        got = O.indexer_topk(bf16_bits(qv)[None, None], wv[None, None], bf16_bits(kv)[None],
                             "bf16", None, q_start=p, kv_len=n, k=k)
        assert got[0, 0].tolist() == _brute_topk(ref, k)


def _loop_scores(qv, wv, kv, n):
    """score[s] for s < n by explicit loops (qv [H, d], wv [H], kv [>=n, d])."""
    ref = []
    for s in range(n):
        tot = 0.0
        for h in range(qv.shape[0]):
            dot = sum(float(qv[h, j]) * float(kv[s, j]) for j in range(qv.shape[1]))
            tot += float(wv[h]) * (dot if dot > 0 else 0.0)
        ref.append(tot)
    return ref


def test_varlen_batch_brute_force_tiny():
    """Sequences of different lengths in one batch: row t of sequence b sits
    at its own start + t and selects among that many + 1 keys of its own
    sequence; checked row by row against loop-summed scores and the
    subset-enumeration selection."""
    rng = np.random.default_rng(3)
    for _ in range(8):
        B, n_q, H, d = int(rng.integers(2, 4)), int(rng.integers(1, 3)), 2, 3
        starts = [int(x) for x in rng.integers(0, 6, size=B)]
        kv_len = max(starts) + n_q
        qv = rng.integers(-3, 4, size=(B, n_q, H, d)).astype(np.float32)
        kv = rng.integers(-3, 4, size=(B, kv_len, d)).astype(np.float32)
        wv = rng.choice([-1.0, 1.0, 2.0], size=(B, n_q, H)).astype(np.float32)
        k = int(rng.integers(1, 6))
        got = O.indexer_topk(bf16_bits(qv), wv, bf16_bits(kv), "bf16", None, q_start=starts,
                             kv_len=kv_len, k=k)
        for b in range(B):
            for t in range(n_q):
                p = starts[b] + t
                ref = _loop_scores(qv[b, t], wv[b, t], kv[b], p + 1)
                assert got[b, t].tolist() == _brute_topk(ref, k), (starts, b, t)


# ------------------------------------------------------------ closed forms --
def _ix(q, w, keys, q_start, kv_len, k, kd="bf16", scale=None):
    return O.indexer_topk(q, w, keys, kd, scale, q_start, kv_len, k)


def test_k_at_least_candidates_selects_whole_prefix():
    rng = np.random.default_rng(3)
    n, H, d = 40, 3, 8
    q = bf16_bits(rng.integers(-8, 9, (1, n, H, d)))
    w = rng.choice([1.0, 2.0, 4.0], (1, n, H)).astype(np.float32)
    keys = bf16_bits(rng.integers(-8, 9, (1, n, d)))
    idx = _ix(q, w, keys, 0, n, k=n)
    for t in range(n):
        assert idx[0, t].tolist() == list(range(t + 1)) + [-1] * (n - t - 1)


def test_zero_query_keeps_lowest_positions():
    n, H, d, k = 50, 2, 4, 7
    q = bf16_bits(np.zeros((1, 1, H, d)))
    w = np.ones((1, 1, H), np.float32)
    keys = bf16_bits(np.random.default_rng(4).integers(-8, 9, (1, n, d)))
    assert _ix(q, w, keys, n - 1, n, k)[0, 0].tolist() == list(range(k))


def test_increasing_scores_keep_latest_positions():
    n, k = 200, 16
    keys = bf16_bits(np.arange(n, dtype=np.float32)[None, :, None])   # key[s] = s
    q = bf16_bits(np.ones((1, 3, 1, 1)))
    w = np.ones((1, 3, 1), np.float32)
    idx = _ix(q, w, keys, n - 3, n, k)
    for i in range(3):
        p = n - 3 + i
        assert idx[0, i].tolist() == list(range(p - k + 1, p + 1))


def test_decreasing_scores_keep_earliest_positions():
    n, k = 200, 16
    keys = bf16_bits(np.arange(n, dtype=np.float32)[None, :, None])
    q = bf16_bits(np.ones((1, 1, 1, 1)))
    w = -np.ones((1, 1, 1), np.float32)                 # score = -s
    assert _ix(q, w, keys, n - 1, n, k)[0, 0].tolist() == list(range(k))


def test_single_head_nonnegative_reduces_to_matmul():
    rng = np.random.default_rng(5)
    qv = rng.integers(0, 9, (1, 16)).astype(np.float32)
    kv = rng.integers(0, 9, (30, 16)).astype(np.float32)
    s = O.indexer_scores(O.decode_bf16(bf16_bits(qv)), np.ones(1), O.key_matrix(bf16_bits(kv), "bf16"))
    np.testing.assert_array_equal(s, (kv.astype(np.float64) @ qv[0].astype(np.float64)))


def test_positive_homogeneity_leaves_selection_unchanged():
    rng = np.random.default_rng(6)
    n, H, d, k = 120, 4, 8, 10
    q = rng.integers(-8, 9, (1, 8, H, d)).astype(np.float32)
    w = rng.choice([1.0, 2.0, 4.0], (1, 8, H)).astype(np.float32)
    keys = bf16_bits(rng.integers(-8, 9, (1, n, d)))
    base = _ix(bf16_bits(q), w, keys, n - 8, n, k)
    assert np.array_equal(base, _ix(bf16_bits(4 * q), w, keys, n - 8, n, k))
    assert np.array_equal(base, _ix(bf16_bits(q), 8 * w, keys, n - 8, n, k))


def test_fp8_keys_with_scale_match_equal_bf16_values():
    """The same key values stored as e4m3fn codes * scale or as bf16 give the
    same selection; the row scale multiplies the key."""
    rng = np.random.default_rng(7)
    n, H, d, k = 64, 4, 16, 9
    ints = rng.integers(-8, 9, (1, n, d)).astype(np.float32)
    codes = torch.from_numpy(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scale = np.full((1, n), 0.125, np.float32)
    q = bf16_bits(rng.integers(-8, 9, (1, 4, H, d)))
    w = rng.choice([1.0, 2.0, 4.0], (1, 4, H)).astype(np.float32)
    a = _ix(q, w, codes, n - 4, n, k, kd="fp8", scale=scale)
    b = _ix(q, w, bf16_bits(ints / 8.0), n - 4, n, k)
    assert np.array_equal(a, b)
    km = O.key_matrix(codes[0], "fp8", scale[0])
    np.testing.assert_array_equal(km, ints[0] / 8.0)


# -------------------------------------------------------------- attention --
def _rand_bf16(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_attention_with_full_prefix_equals_dense_causal_sdpa():
    """k >= candidate count: sparse attention over the whole prefix must equal
    dense causal attention (torch's scaled_dot_product_attention, float64)."""
    rng = np.random.default_rng(8)
    L, Hq, D, Dv = 12, 3, 8, 5
    Q = _rand_bf16(rng, (1, L, Hq, D))
    KV = _rand_bf16(rng, (1, L, D))
    idx = np.full((1, L, L), -1, np.int32)
    for t in range(L):
        idx[0, t, : t + 1] = np.arange(t + 1)
    sm = 1.0 / math.sqrt(D)
    o, lse = O.sparse_attention(Q, KV, idx, L, sm, Dv)
    q = torch.from_numpy(O.decode_bf16(Q[0])).permute(1, 0, 2)[None]          # [1,Hq,L,D]
    kvt = torch.from_numpy(O.decode_bf16(KV[0]))
    kk = kvt[None, None].expand(1, Hq, L, D)
    vv = kvt[None, None, :, :Dv].expand(1, Hq, L, Dv)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True, scale=sm)
    np.testing.assert_allclose(o[0], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # lse against a log-sum-exp over the causal logits
    logits = (q @ kk.transpose(-1, -2)) * sm
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), 1)
    ref_lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), dim=-1)   # [1,Hq,L]
    np.testing.assert_allclose(lse[0], ref_lse[0].T.numpy(), rtol=0, atol=1e-12)


def test_attention_single_slot_returns_value_row():
    rng = np.random.default_rng(9)
    Q = _rand_bf16(rng, (1, 1, 4, 16))
    KV = _rand_bf16(rng, (1, 10, 16))
    idx = np.full((1, 1, 6), -1, np.int32)
    idx[0, 0, 3] = 7
    o, _ = O.sparse_attention(Q, KV, idx, 10, 0.3, 12)
    for h in range(4):
        np.testing.assert_array_equal(o[0, 0, h], O.decode_bf16(KV[0, 7, :12]))


def test_attention_zero_query_is_mean_of_selected_values():
    rng = np.random.default_rng(10)
    Q = bf16_bits(np.zeros((1, 1, 2, 8)))
    KV = _rand_bf16(rng, (1, 20, 8))
    sel = [2, 5, 11, 19]
    idx = np.asarray([[sel + [-1, -1]]], np.int32)
    o, lse = O.sparse_attention(Q, KV, idx, 20, 1.0, 6)
    ref = O.decode_bf16(KV[0, sel, :6]).mean(axis=0)
    np.testing.assert_allclose(o[0, 0, 0], ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], math.log(4.0), rtol=0, atol=1e-15)


def test_attention_ignores_out_of_range_slots_and_slot_order():
    rng = np.random.default_rng(11)
    Q = _rand_bf16(rng, (1, 1, 2, 8))
    KV = _rand_bf16(rng, (1, 20, 8))
    a = np.asarray([[[1, 4, 9, -1, -1]]], np.int32)
    b = np.asarray([[[9, -1, 1, 25, 4]]], np.int32)      # 25 >= kv_len: ignored
    oa, la = O.sparse_attention(Q, KV, a, 20, 0.5, 8)
    ob, lb = O.sparse_attention(Q, KV, b, 20, 0.5, 8)
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-14)
    none = np.full((1, 1, 3), -1, np.int32)
    on, ln = O.sparse_attention(Q, KV, none, 20, 0.5, 8)
    assert np.all(on == 0) and np.all(np.isneginf(ln))


# --------------------------------------------------------------- schedule --
def _group_inputs(rng, roles, n=24, H=2, d=4, Hq=2, D=8, same_indexer=False):
    ixl, atl = [], []
    shared = None
    for _ in roles:
        if same_indexer and shared is not None:
            ixl.append(shared)
        else:
            q = bf16_bits(rng.integers(-8, 9, (1, n, H, d)))
            w = rng.choice([1.0, 2.0, 4.0], (1, n, H)).astype(np.float32)
            keys = bf16_bits(rng.integers(-8, 9, (1, n, d)))
            shared = (q, w, keys, "bf16", None)
            ixl.append(shared)
        atl.append((_rand_bf16(rng, (1, n, Hq, D)), _rand_bf16(rng, (1, n, D))))
    return ixl, atl


def test_schedule_fsss_runs_indexer_once_and_shares_positions():
    rng = np.random.default_rng(12)
    ixl, atl = _group_inputs(rng, "FSSS")
    r = O.group_forward("FSSS", ixl, atl, 0, 24, 5, 0.35, 6)
    assert r["n_indexer_runs"] == 1 and r["used"] == [0, 0, 0, 0] and len(r["idx"]) == 1
    for l in range(4):     # every layer attends over exactly the F layer's positions
        o, _ = O.sparse_attention(atl[l][0], atl[l][1], r["idx"][0], 24, 0.35, 6)
        np.testing.assert_array_equal(o, r["O"][l])
    assert not np.array_equal(r["O"][0], r["O"][1])   # own Q/KV per layer


def test_schedule_two_groups_and_all_full_equivalence():
    rng = np.random.default_rng(13)
    ixl, atl = _group_inputs(rng, "FSSSFSSS")
    r = O.group_forward("FSSSFSSS", ixl, atl, 0, 24, 5, 0.35, 6)
    assert r["n_indexer_runs"] == 2 and r["used"] == [0] * 4 + [1] * 4
    # all-F with identical indexer inputs per group reproduces F+3S
    ix_same = [ixl[0]] * 4 + [ixl[4]] * 4
    rf = O.group_forward("FFFFFFFF", ix_same, atl, 0, 24, 5, 0.35, 6)
    assert rf["n_indexer_runs"] == 8
    for l in range(8):
        np.testing.assert_array_equal(rf["O"][l], r["O"][l])


def test_schedule_rejects_leading_shared_layer():
    rng = np.random.default_rng(14)
    ixl, atl = _group_inputs(rng, "SFSS")
    with pytest.raises(ValueError):
        O.group_forward("SFSS", ixl, atl, 0, 24, 5, 0.35, 6)


def test_mtp_draft_later_steps_attend_over_the_first_steps_prefix():
    """MTP draft steps: the first step selects with k >= its candidate count,
    so it keeps the whole prefix 0..pos; the cache already holds the rows of
    the later draft tokens (kv_len = pos + steps), yet every step must equal
    dense attention over rows 0..pos only (torch's scaled_dot_product_attention
    in float64), and the indexer runs once."""
    rng = np.random.default_rng(16)
    pos, steps, Hq, D, Dv, H, d = 9, 4, 2, 8, 6, 2, 4
    kv_len = pos + steps
    q = bf16_bits(rng.integers(-8, 9, (1, 1, H, d)))
    w = rng.choice([1.0, 2.0], (1, 1, H)).astype(np.float32)
    keys = bf16_bits(rng.integers(-8, 9, (1, kv_len, d)))
    KV = _rand_bf16(rng, (1, kv_len, D))
    drafts = [_rand_bf16(rng, (1, 1, Hq, D)) for _ in range(steps)]
    sm = 0.4
    r = O.mtp_draft((q, w, keys, "bf16", None), drafts, KV, pos, kv_len, 16, sm, Dv)
    assert r["n_indexer_runs"] == 1 and len(r["O"]) == steps
    assert r["idx"][0, 0].tolist() == list(range(pos + 1)) + [-1] * (16 - pos - 1)
    kvt = torch.from_numpy(O.decode_bf16(KV[0, : pos + 1]))
    for j in range(steps):
        qq = torch.from_numpy(O.decode_bf16(drafts[j][0, 0]))[None, :, None, :]     # [1,Hq,1,D]
        kk = kvt[None, None].expand(1, Hq, pos + 1, D)
        vv = kvt[None, None, :, :Dv].expand(1, Hq, pos + 1, Dv)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=sm)
        np.testing.assert_allclose(r["O"][j][0, 0], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_oracle_exports():
    for name in oracle.__all__:
        assert callable(getattr(oracle, name))


def test_row_form_agrees_with_batch_form():
    """indexer_topk_rows (rows given by absolute position) and indexer_topk
    (rows given by index) compute the same rows."""
    rng = np.random.default_rng(15)
    n, H, d, k = 90, 3, 8, 11
    q = bf16_bits(rng.integers(-8, 9, (1, 30, H, d)))
    w = rng.choice([1.0, 2.0, 4.0], (1, 30, H)).astype(np.float32)
    keys = bf16_bits(rng.integers(-8, 9, (1, n, d)))
    full = O.indexer_topk(q, w, keys, "bf16", None, 60, n, k)
    rows = [0, 7, 29]
    part = O.indexer_topk_rows(q[0, rows], w[0, rows], keys[0], "bf16", None, [60 + r for r in rows], n, k)
    np.testing.assert_array_equal(part, full[0, rows])


# ------------------------------------------------------------ index overlap --
def _row(vals, k):
    r = np.full(k, -1, dtype=np.int32)
    r[:len(vals)] = sorted(vals)
    return r


def test_overlap_identical_rows_count_valid_slots():
    """Closed form: a row overlaps itself in exactly its valid slots."""
    rng = np.random.default_rng(3)
    rows = [_row(rng.choice(5000, size=n, replace=False), 64) for n in (0, 1, 17, 64)]
    a = np.stack(rows)
    np.testing.assert_array_equal(O.index_overlap(a, a), [0, 1, 17, 64])


def test_overlap_shifted_ranges_closed_form():
    """[0, n) against [m, m + n): max(0, n - m) common positions."""
    k = 32
    for n, m in ((32, 0), (32, 5), (20, 19), (20, 20), (20, 31), (7, 3)):
        a = _row(range(n), k)[None]
        b = _row(range(m, m + n), k)[None]
        assert O.index_overlap(a, b)[0] == max(0, n - m)


def test_overlap_ignores_padding_and_is_symmetric():
    """-1 padding never counts even when both rows are padded in the same
    slots; the count is symmetric in its arguments."""
    a = np.array([[2, 5, 9, -1, -1], [-1, -1, -1, -1, -1]], dtype=np.int32)
    b = np.array([[5, 9, 11, -1, -1], [-1, -1, -1, -1, -1]], dtype=np.int32)
    np.testing.assert_array_equal(O.index_overlap(a, b), [2, 0])
    np.testing.assert_array_equal(O.index_overlap(b, a), [2, 0])


def test_overlap_keeps_leading_shape():
    a = np.zeros((2, 3, 4), dtype=np.int32)
    assert O.index_overlap(a, a).shape == (2, 3)
    with pytest.raises(ValueError):
        O.index_overlap(a, a[:, :2])


# ------------------------------------------------------------ key quantizing --
def test_e4m3fn_encode_matches_torch_on_grid_and_midpoints():
    """The encoder agrees with torch's float8_e4m3fn conversion (a library
    routine) on every code value, on the exact midpoints between neighbouring
    codes (ties to the even code), just beside them, on subnormals, and
    saturates like torch after clamping to +-448."""
    codes = np.arange(256, dtype=np.uint8)
    vals = O.decode_e4m3fn(codes)
    fin = np.sort(np.unique(vals[~np.isnan(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2
    eps = np.abs(mids) * 1e-6 + 1e-12
    xs = np.concatenate([fin, mids, mids + eps, mids - eps, [500.0, -1e6, 448.001, -448.001, 1e-9, -1e-9]])
    xs = xs.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(np.clip(xs, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    got = O.encode_e4m3fn(xs)
    # the two zeros decode alike; compare values where the sign of zero differs
    np.testing.assert_array_equal(O.decode_e4m3fn(got), O.decode_e4m3fn(ref))


def test_quantize_rows_closed_forms():
    """A row of one repeated magnitude v maps to +-448 codes with scale v/448;
    an all-zero row gets scale 1 and zero codes; the largest magnitude of any
    row always lands exactly on +-448."""
    rows = np.array([[3.0, -3.0, 3.0, 3.0], [0.0, 0.0, 0.0, 0.0], [28.0, -14.0, 7.0, 3.5]], dtype=np.float32)
    codes, scale = O.quantize_key_rows(rows)
    assert scale[0] == np.float32(3.0) / np.float32(448.0)
    np.testing.assert_array_equal(O.decode_e4m3fn(codes[0]), [448.0, -448.0, 448.0, 448.0])
    assert scale[1] == 1.0 and np.all(O.decode_e4m3fn(codes[1]) == 0.0)
    assert O.decode_e4m3fn(codes[2])[0] == 448.0
    # amax 28 gives the power-of-two scale 1/16: decoded codes times it
    # reproduce the row exactly
    np.testing.assert_array_equal(O.decode_e4m3fn(codes[2]) * scale[2], rows[2].astype(np.float64))


def test_quantize_rows_error_bound():
    """Each decoded value is within half a code step (relative 2^-4 for
    normals) of the scaled input: e4m3fn has 3 mantissa bits."""
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((64, 128)).astype(np.float32)
    codes, scale = O.quantize_key_rows(rows)
    y = rows / scale[:, None].astype(np.float64)
    back = O.decode_e4m3fn(codes)
    tol = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(back - y) <= tol)


# ------------------------------------------------- indexer inputs (f1 opt) --
def test_bf16_encode_matches_torch_on_random_values_and_midpoints():
    """encode_bf16 (round to nearest, ties to even) against torch's float32 ->
    bfloat16 conversion: random float32 values over many binades, the exact
    midpoints between neighbouring bf16 values, and the floats just beside
    them."""
    rng = np.random.default_rng(11)
    mags = np.ldexp(rng.uniform(1.0, 2.0, 4000), rng.integers(-60, 60, 4000))
    v = (mags * rng.choice([-1.0, 1.0], 4000)).astype(np.float32)
    lo = O.decode_bf16(O.encode_bf16(v.astype(np.float64)))          # some bf16 values
    ulp = np.ldexp(1.0, np.frexp(lo)[1] - 8)
    mid = (lo + 0.5 * ulp).astype(np.float32)                          # exact in float32
    beside = np.concatenate([np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))])
    for vals in (v, mid, beside.astype(np.float32)):
        got = O.encode_bf16(vals.astype(np.float64))
        ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(got, ref)


def test_hand_worked_projection():
    g = gold()["project"]
    x = np.asarray(g["x"], dtype=np.float64)
    w = np.asarray(g["w_proj"], dtype=np.float64)
    q, wt = O.indexer_project(O.encode_bf16(x), O.encode_bf16(w), g["heads"], g["dim"])
    np.testing.assert_array_equal(O.decode_bf16(q), np.asarray(g["q"]))
    np.testing.assert_array_equal(wt, np.asarray(g["w"]))


def test_projection_one_hot_rows_select_weight_columns():
    """x = e_j picks column j of W: every output is a stored bf16 weight, so
    q reproduces its bit pattern and w its value."""
    rng = np.random.default_rng(5)
    H, d, d_in = 3, 4, 16
    wb = O.encode_bf16(rng.normal(size=(H * d + H, d_in)))
    xb = O.encode_bf16(np.eye(d_in))
    q, wt = O.indexer_project(xb, wb, H, d)
    np.testing.assert_array_equal(q.reshape(d_in, H * d), wb[: H * d].T)
    np.testing.assert_array_equal(wt, O.decode_bf16(wb[H * d:]).T)


def test_projection_rounds_midpoints_to_even():
    """x = [1, 2^-8]: W row [1, 1] gives 1 + 2^-8, halfway between 1 and
    1 + 2^-7, which rounds to 1 (even pattern); W row [1, 3] gives
    1 + 3*2^-8, halfway between 1 + 2^-7 and 1 + 2^-6, which rounds up to
    1 + 2^-6; the head-weight column [2, 0] stays 2."""
    xb = O.encode_bf16(np.array([[1.0, 2.0 ** -8]]))
    wb = O.encode_bf16(np.array([[1.0, 1.0], [1.0, 3.0], [2.0, 0.0]]))
    q, wt = O.indexer_project(xb, wb, 1, 2)
    np.testing.assert_array_equal(O.decode_bf16(q)[0, 0], [1.0, 1.0 + 2.0 ** -6])
    np.testing.assert_array_equal(wt, [[2.0]])


def test_projection_head_weights_scale_exactly():
    """Scaling x by a power of two scales the head weights exactly (and q up
    to its own rounding, which a power of two does not change)."""
    rng = np.random.default_rng(9)
    H, d, d_in = 2, 4, 32
    wb = O.encode_bf16(rng.normal(size=(H * d + H, d_in)))
    x = rng.normal(size=(5, d_in))
    q1, w1 = O.indexer_project(O.encode_bf16(x), wb, H, d)
    q2, w2 = O.indexer_project(O.encode_bf16(4.0 * O.decode_bf16(O.encode_bf16(x))), wb, H, d)
    np.testing.assert_array_equal(w2, 4.0 * w1)
    np.testing.assert_array_equal(O.decode_bf16(q2), 4.0 * O.decode_bf16(q1))


def test_hand_worked_fp8_queries():
    """e4m3fn-coded queries times their (row, head) scale (IndexCache notes,
    section 1: an FP8 indexer), worked by hand in the golden file."""
    c = gold()["fp8_queries"]
    q = O.query_matrix(np.array(c["q_codes"], dtype=np.uint8), np.array(c["q_scale"]))
    np.testing.assert_array_equal(q, [[3.0, -4.0], [0.125, 1.0]])
    s = O.indexer_scores(q, np.array(c["w"], dtype=np.float64), np.array(c["keys"], dtype=np.float64))
    np.testing.assert_array_equal(s, c["scores"])


def _e4m3_code_of(values):
    """Codes of e4m3fn-representable values, found by inverting the (pinned)
    decode table over all 256 codes."""
    table = {float(v): c for c, v in enumerate(O.decode_e4m3fn(np.arange(256, dtype=np.uint8)))
             if np.isfinite(v) and not (v == 0.0 and c != 0)}
    return np.vectorize(lambda v: table[float(v)], otypes=[np.uint8])(values)


def test_fp8_queries_with_power_of_two_scales_match_bf16_values():
    """Queries whose values are e4m3fn codes times a power of two per (row,
    head) are exactly bf16 values too: both query forms give the same scores
    and the same top-k."""
    rng = np.random.default_rng(7)
    B, n_q, H, d, L, k = 1, 6, 3, 8, 40, 9
    ints = rng.integers(-8, 9, (B, n_q, H, d)).astype(np.float64)
    scale = np.ldexp(1.0, rng.integers(-3, 4, (B, n_q, H))).astype(np.float32)
    codes = _e4m3_code_of(ints)
    vals = ints * scale[..., None].astype(np.float64)
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(O.decode_bf16(bits), vals)
    w = rng.standard_normal((B, n_q, H)).astype(np.float32)
    keys = (rng.standard_normal((B, L, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    a = O.indexer_topk(bits, w, keys, "bf16", None, L - n_q, L, k)
    b = O.indexer_topk(codes, w, keys, "bf16", None, L - n_q, L, k, q_scale=scale)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(O.query_matrix(codes, scale), vals)
