"""GPU parity of ix_indexer_argmax, the top-1 of the indexer scores (the fused
kernel with a running maximum in place of the streaming top-k), against the
CPU oracle's scores and its k = 1 selection rule ("IndexShare", LLM
Architecture Gallery, section "Why The Indexer Becomes Expensive").

Exact-mode inputs make every fp32 partial sum exact, so positions and scores
must match bit for bit; float-mode rows are compared by position, and where
the two sides pick different positions the oracle must rate both as a
near-tie."""
import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes
import ix_synth as synth
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _run(ix, w, inputs=None, seq=None):
    if inputs is None:
        q, wt = synth.indexer_queries(w, "cuda", 0)
        keys, scale = synth.indexer_keys(w, "cuda", 0)
        inputs = (q, wt, keys, scale)
    q, wt, keys, scale = inputs
    pos = torch.full((w.batch, w.n_q), -7, dtype=torch.int32, device="cuda")
    score = torch.full((w.batch, w.n_q), float("nan"), device="cuda")
    print(f"[argmax] {w.name} B={w.batch} n_q={w.n_q} q_start={w.q_start} kv_len={w.kv_len} "
          f"H={w.ix_heads} d={w.ix_dim} keys={w.key_dtype} mode={w.mode} varlen={seq is not None}", flush=True)
    ix.ix_indexer_argmax(q, wt, keys, pos, score, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len,
                         seq_q_start=seq)
    torch.cuda.synchronize()
    return inputs, host(pos), host(score)


def _oracle_rows(w, inputs, b, rows, start):
    """Oracle scores of the listed rows of sequence b: (best position under
    the k = 1 rule, full score vector) per row."""
    q, wt, keys, scale = inputs
    kb, kd = key_bytes(keys[b:b + 1])
    sc = None if scale is None else host(scale[b])
    p_max = min(start + max(rows), w.kv_len - 1)
    kmat = O.key_matrix(kb[0, : p_max + 1], kd, None if sc is None else sc[: p_max + 1])
    qb, wb = bits16(q[b]), host(wt[b])
    out = []
    for t in rows:
        n = min(start + t, w.kv_len - 1) + 1
        s = O.indexer_scores(O.decode_bf16(qb[t]), np.asarray(wb[t], np.float64), kmat[:n])
        out.append((int(O.select_topk(s, 1)[0]), s))
    return out


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("heads,dim", [(64, 128), (5, 32), (33, 64), (7, 16)])
def test_exact_bit_exact(ix, key_dtype, heads, dim):
    """Integer inputs: positions (ties -> lower) and scores bit for bit, over
    ragged tiles, a partial last row block and a chunk that starts mid-way."""
    w = synth.L16K.with_(name=f"argmax_exact_{key_dtype}_{heads}x{dim}", batch=2, n_q=777, q_start=1500,
                         kv_len=2400, ix_heads=heads, ix_dim=dim, key_dtype=key_dtype, mode="exact")
    inputs, pos, score = _run(ix, w)
    rows = list(range(0, w.n_q, 5)) + [w.n_q - 1]
    for b in range(w.batch):
        for t, (p_ref, s) in zip(rows, _oracle_rows(w, inputs, b, rows, w.q_start)):
            assert pos[b, t] == p_ref, (b, t)
            assert score[b, t] == s[p_ref], (b, t)


def test_all_equal_scores_pick_position_zero(ix):
    """q = 0: every score is +-0 (negative weights give -0.0), all equal, so
    every row's best is position 0 with score 0."""
    w = synth.L16K.with_(name="argmax_ties", n_q=500, kv_len=500, ix_heads=64, ix_dim=128)
    q, wt = synth.indexer_queries(w, "cuda", 0)
    keys, _ = synth.indexer_keys(w, "cuda", 0)
    _, pos, score = _run(ix, w, (torch.zeros_like(q), wt, keys, None))
    assert np.all(pos == 0)
    assert np.all(score == 0.0)


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
def test_float_rows(ix, key_dtype):
    """Float inputs: the same position as the oracle in >= 99.9% of rows; a
    different pick must be a near-tie in the oracle's float64 scores, and the
    GPU's fp32 score is within rounding of the oracle's best."""
    w = synth.L16K.with_(name=f"argmax_float_{key_dtype}", n_q=2000, kv_len=2000, key_dtype=key_dtype)
    inputs, pos, score = _run(ix, w)
    rows = list(range(0, w.n_q, 3))
    same = 0
    for t, (p_ref, s) in zip(rows, _oracle_rows(w, inputs, 0, rows, 0)):
        best = s[p_ref]
        tol = 1e-5 * np.abs(s).max() + 1e-6
        assert abs(float(score[0, t]) - best) <= tol, (t, score[0, t], best)
        if pos[0, t] == p_ref:
            same += 1
        else:
            assert 0 <= pos[0, t] <= t and best - s[pos[0, t]] <= tol, (t, pos[0, t], p_ref)
    assert same / len(rows) >= 0.999


def test_sequences_of_different_lengths(ix):
    """Per-sequence starts read on the device: each sequence's rows select
    among its own positions, bit for bit in exact mode."""
    w = synth.L16K.with_(name="argmax_varlen", batch=3, n_q=300, q_start=2000, kv_len=2300,
                         key_dtype="fp8", mode="exact")
    starts = [2000, 0, 777]
    seq = torch.tensor(starts, dtype=torch.int64, device="cuda")
    inputs, pos, score = _run(ix, w, seq=seq)
    rows = list(range(0, w.n_q, 7)) + [w.n_q - 1]
    for b in range(w.batch):
        for t, (p_ref, s) in zip(rows, _oracle_rows(w, inputs, b, rows, starts[b])):
            assert pos[b, t] == p_ref and score[b, t] == s[p_ref], (b, t)


def test_argmax_equals_topk_with_k1(ix):
    """The running-max kernel and the streaming top-k with k = 1 agree."""
    w = synth.L16K.with_(name="argmax_vs_topk1", n_q=1500, kv_len=1500, k=1, key_dtype="fp8")
    inputs, pos, _ = _run(ix, w)
    q, wt, keys, scale = inputs
    idx = torch.empty((1, w.n_q, 1), dtype=torch.int32, device="cuda")
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=0, kv_len=w.kv_len, path=ix.IX_PATH_FUSED)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx)[0, :, 0], pos[0])
