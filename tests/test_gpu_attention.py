"""GPU parity of the sparse gather attention against the CPU oracle, given
identical indices (max-abs error <= 2e-2 on the bf16 outputs)."""
import math

import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host
import ix_synth as synth
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-2


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _attn(ix, w, Q, KV, idx, splits=0, sm_scale=0.0):
    out = torch.full((w.batch, w.n_q, w.q_heads, w.d_v), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((w.batch, w.n_q, w.q_heads), float("nan"), device="cuda")
    print(f"[attn] {w.name} B={w.batch} n_q={w.n_q} kv_len={w.kv_len} k={idx.shape[-1]} "
          f"Hq={w.q_heads} D={w.d_qk} Dv={w.d_v} splits={splits}", flush=True)
    ix.ix_sparse_attn(Q, KV, idx, out, lse=lse, q_start=w.q_start, kv_len=w.kv_len,
                      sm_scale=sm_scale, kv_splits=splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), host(lse)


def _oracle(w, Q, KV, idx, rows, sm_scale=None):
    sm = sm_scale if sm_scale else 1.0 / math.sqrt(w.d_qk)
    return O.sparse_attention(bits16(Q), bits16(KV), host(idx), w.kv_len, sm, w.d_v, rows=rows)


def _indices(ix, w):
    q, wt = synth.indexer_queries(w, "cuda")
    keys, scale = synth.indexer_keys(w, "cuda")
    idx = torch.empty((w.batch, w.n_q, w.k), dtype=torch.int32, device="cuda")
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len)
    return idx


def _check(got, lse, ref, ref_lse, rows):
    o = got[:, rows]
    err = np.abs(o - ref).max()
    print(f"max abs err {err:.3e}")
    assert err <= ATOL
    np.testing.assert_allclose(lse[:, rows], ref_lse, rtol=0, atol=1e-3)


def test_tiny_config_all_rows(ix):
    w = synth.TINY_L1K
    idx = _indices(ix, w)
    Q, KV = synth.attn_queries(w, "cuda", 0), synth.latent_kv(w, "cuda", 0)
    got, lse = _attn(ix, w, Q, KV, idx)
    rows = list(range(w.n_q))
    ref, ref_lse = _oracle(w, Q, KV, idx, rows)
    _check(got, lse, ref, ref_lse, rows)


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_latent_576_k2048_ragged(ix, splits):
    """MLA latent rows (576 = 512 V + 64 rope), 16 heads, k = 2048, rows with
    fewer than k candidates padded with -1, ragged slot splits."""
    w = synth.L16K.with_(name="attn_l3000", n_q=3000, kv_len=3000)
    idx = _indices(ix, w)
    Q, KV = synth.attn_queries(w, "cuda", 1), synth.latent_kv(w, "cuda", 1)
    got, lse = _attn(ix, w, Q, KV, idx, splits=splits)
    rows = [0, 1, 2, 17, 500, 2046, 2047, 2048, 2049, 2999]
    ref, ref_lse = _oracle(w, Q, KV, idx, rows)
    _check(got, lse, ref, ref_lse, rows)


def test_holes_out_of_range_and_duplicates(ix):
    """Arbitrary slot contents: -1 holes anywhere, entries >= kv_len ignored,
    duplicated positions counted twice, an empty row -> zeros / -inf."""
    w = synth.L16K.with_(name="attn_holes", batch=2, n_q=40, kv_len=900, kv_cap=1000, k=200)
    g = torch.Generator(device="cuda").manual_seed(3)
    idx = torch.randint(-1, 1000, (2, 40, 200), generator=g, device="cuda", dtype=torch.int32)
    idx[:, :, 5] = idx[:, :, 9]
    idx[1, 7] = -1
    Q = synth.attn_queries(w, "cuda", 2)
    KV = synth.latent_kv(w, "cuda", 2)
    for splits in (1, 4):
        got, lse = _attn(ix, w, Q, KV, idx, splits=splits)
        assert np.all(got[1, 7] == 0) and np.all(np.isneginf(lse[1, 7]))
        rows = list(range(40))
        ref, ref_lse = _oracle(w, Q, KV, idx, rows)
        assert np.abs(got - ref).max() <= ATOL
        fin = np.isfinite(ref_lse)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=0, atol=1e-3)


def test_single_slot_returns_value_row_exactly(ix):
    w = synth.L16K.with_(name="attn_single", n_q=8, kv_len=64, k=32)
    idx = torch.full((1, 8, 32), -1, dtype=torch.int32, device="cuda")
    for t in range(8):
        idx[0, t, (3 * t) % 32] = 5 * t
    Q, KV = synth.attn_queries(w, "cuda", 3), synth.latent_kv(w, "cuda", 3)
    got, _ = _attn(ix, w, Q, KV, idx)
    kv = KV.float().cpu().numpy()
    for t in range(8):
        for h in range(w.q_heads):
            np.testing.assert_array_equal(got[0, t, h], kv[0, 5 * t, : w.d_v])


def test_full_prefix_equals_dense_causal(ix):
    """k >= candidate count: sparse attention over idx = [0..p] equals dense
    causal attention (compared through the oracle, which is pinned to torch's
    scaled_dot_product_attention)."""
    w = synth.TINY_L1K.with_(name="dense_eq", n_q=300, kv_len=300, k=304)
    idx = torch.full((1, 300, 304), -1, dtype=torch.int32, device="cuda")
    for t in range(300):
        idx[0, t, : t + 1] = torch.arange(t + 1, device="cuda", dtype=torch.int32)
    Q, KV = synth.attn_queries(w, "cuda", 4), synth.latent_kv(w, "cuda", 4)
    got, lse = _attn(ix, w, Q, KV, idx, sm_scale=0.125)
    rows = list(range(300))
    ref, ref_lse = _oracle(w, Q, KV, idx, rows, sm_scale=0.125)
    _check(got, lse, ref, ref_lse, rows)


@pytest.mark.parametrize("n_q", [4, 1024])
def test_dominant_logit_in_every_key_group(ix, n_q):
    """One slot per row has logit 256 (natural units) and the others 0, so the
    output is that slot's value row exactly and lse = 256.  The dominant slot
    sits in a different one of the four 4-key groups of a 16-slot step (and,
    with few rows, in a different wave of the four sharing a row) from row to
    row: a running max that missed a group would leave 2^369 unscaled and
    overflow.  n_q = 4 runs the four-waves-per-row split, 1024 one wave per
    row."""
    k, L = 64, 2048
    w = synth.TINY_L1K.with_(name="dominant", n_q=n_q, q_start=L - n_q, kv_len=L, k=k, q_heads=8, d_qk=128,
                             d_v=96)
    KV = torch.zeros((1, L, w.d_qk), dtype=torch.bfloat16, device="cuda")
    KV[0, :, 1:] = torch.randn((L, w.d_qk - 1), generator=torch.Generator(device="cuda").manual_seed(3),
                               device="cuda").to(torch.bfloat16)
    dom = 1000 + torch.arange(16, device="cuda")
    KV[0, dom, 0] = 16.0
    Q = torch.zeros((1, n_q, w.q_heads, w.d_qk), dtype=torch.bfloat16, device="cuda")
    Q[..., 0] = 16.0
    r = torch.arange(n_q, device="cuda")
    idx = torch.arange(k, dtype=torch.int32, device="cuda").repeat(1, n_q, 1)
    slot = 16 * (r % 4) + 4 * ((r + r // 4) % 4) + (r % 3)       # wave r%4; rows 0..3 cover groups 0..3
    idx[0, r, slot] = dom[(r % 16)].to(torch.int32)
    got, lse = _attn(ix, w, Q, KV, idx, sm_scale=1.0)
    want = KV[0, dom[(r % 16)], : w.d_v].float().cpu().numpy()          # [n_q, Dv]
    assert np.isfinite(got).all() and np.isfinite(lse).all()
    np.testing.assert_array_equal(got[0], np.broadcast_to(want[:, None, :], got[0].shape))
    np.testing.assert_allclose(lse[0], 256.0, rtol=0, atol=1e-3)
