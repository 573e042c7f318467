"""Batches of sequences of different lengths (a per-sequence start of the
query rows, ix_problem.seq_q_start) against the CPU oracle, through every
entry point that reads positions: the indexer on both paths, the row top-k,
the layer group and the key append.  Integer-valued inputs keep the selected
positions bit-exact."""
import math

import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes, valid_idx_rows
import ix_synth as synth
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

PATHS = [1, 2]          # fused streaming, materialised scores


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _dev_starts(starts):
    return torch.tensor(starts, dtype=torch.int64, device="cuda")


def _indexer(ix, w, starts, path, inputs=None, bound=None):
    if inputs is None:
        q, wt = synth.indexer_queries(w, "cuda", 0)
        keys, scale = synth.indexer_keys(w, "cuda", 0)
        inputs = (q, wt, keys, scale)
    q, wt, keys, scale = inputs
    idx = torch.full((w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[varlen] {w.name} B={w.batch} n_q={w.n_q} starts={starts} bound={bound} kv_len={w.kv_len} "
          f"k={w.k} keys={w.key_dtype} path={path}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=bound, kv_len=w.kv_len, path=path,
                       seq_q_start=_dev_starts(starts))
    torch.cuda.synchronize()
    return inputs, host(idx)


def _oracle(w, inputs, starts, rows):
    q, wt, keys, scale = inputs
    kb, kd = key_bytes(keys)
    return O.indexer_topk(bits16(q), host(wt), kb, kd, host(scale), starts, w.kv_len, w.k, rows=rows)


def _valid_per_sequence(got, starts, k):
    for b, s in enumerate(starts):
        valid_idx_rows(got[b:b + 1], s, k)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
def test_exact_prefill_chunks_of_different_starts(ix, path, key_dtype):
    """Four sequences whose 260-row query blocks start at 0, 1700, 333 and
    2900: rows below and above k, the largest start equal to the bound."""
    starts = [0, 1700, 333, 2900]
    w = synth.L16K.with_(name="exact_varlen", batch=4, n_q=260, q_start=2900, kv_len=3160, k=512,
                         mode="exact", key_dtype=key_dtype)
    inputs, got = _indexer(ix, w, starts, path)
    _valid_per_sequence(got, starts, w.k)
    rows = [0, 1, 2, 3, 100, 179, 180, 255, 258, 259]
    np.testing.assert_array_equal(got[:, rows], _oracle(w, inputs, starts, rows))


def test_exact_decode_rows_of_different_lengths(ix):
    """Decode in miniature: eight sequences, one query each, contexts from 1
    key to 40,001 keys (below, at and above k = 2048); fp8 keys, materialised
    scores and the multi-workgroup row select."""
    starts = [40000, 0, 2046, 2047, 2048, 12345, 39999, 777]
    w = synth.DECODE_B32.with_(name="decode_varlen", batch=8, q_start=40000, kv_len=40001, kv_cap=40064,
                               mode="exact")
    inputs, got = _indexer(ix, w, starts, 0)
    _valid_per_sequence(got, starts, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs, starts, None))


@pytest.mark.parametrize("path", PATHS)
def test_out_of_range_starts_are_clamped(ix, path):
    """Entries below 0 or above the bound act as 0 and the bound."""
    w = synth.L16K.with_(name="clamp_varlen", batch=3, n_q=200, q_start=1000, kv_len=1200, k=256,
                         mode="exact")
    inputs, got = _indexer(ix, w, [-5, 10 ** 12, 400], path, bound=w.q_start)
    rows = [0, 1, 57, 199]
    np.testing.assert_array_equal(got[:, rows], _oracle(w, inputs, [0, 1000, 400], rows))


def test_equal_starts_match_the_common_start(ix):
    """A per-sequence array holding the common start changes nothing."""
    w = synth.L16K.with_(name="same_varlen", batch=2, n_q=300, q_start=900, kv_len=1200, k=256,
                         mode="exact", key_dtype="fp8")
    inputs, got = _indexer(ix, w, [900, 900], 0)
    q, wt, keys, scale = inputs
    idx = torch.empty((w.batch, w.n_q, w.k), dtype=torch.int32, device="cuda")
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=900, kv_len=w.kv_len)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, host(idx))


def test_topk_scores_per_sequence_rows(ix):
    g = torch.Generator(device="cuda").manual_seed(6)
    B, n_q, L, k = 3, 4, 5000, 700
    starts = [0, 4996, 2000]
    scores = torch.randint(-40, 40, (B, n_q, L), generator=g, device="cuda").float()
    idx = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    print(f"[varlen] topk_scores B={B} n_q={n_q} L={L} starts={starts}", flush=True)
    ix.ix_topk_scores(scores, idx, kv_len=L, seq_q_start=_dev_starts(starts))
    torch.cuda.synchronize()
    s, got = host(scores), host(idx)
    for b in range(B):
        for t in range(n_q):
            p = starts[b] + t
            np.testing.assert_array_equal(got[b, t], O.select_topk(s[b, t, : p + 1].astype(np.float64), k))


def test_group_forward_with_per_sequence_starts(ix):
    """F,S,S over three sequences of different lengths: each F slot and each
    layer's attention against the oracle's group walk."""
    starts = [0, 500, 260]
    w = synth.TINY_L1K.with_(name="group_varlen", batch=3, n_q=130, q_start=500, kv_len=630, k=64)
    roles = "FSS"
    ixl, atl = [], []
    for l, r in enumerate(roles):
        if r == "F":
            q, wt = synth.indexer_queries(w, "cuda", l)
            keys, scale = synth.indexer_keys(w, "cuda", l)
            ixl.append(dict(q=q, w=wt, keys=keys, k_scale=scale))
        else:
            ixl.append(None)
        atl.append(dict(q=synth.attn_queries(w, "cuda", l), kv=synth.latent_kv(w, "cuda", l),
                        out=torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device="cuda")))
    idx = torch.full((1, w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[varlen] group {roles} starts={starts}", flush=True)
    ix.ix_group_forward(ixl, atl, 1, idx, kv_len=w.kv_len, seq_q_start=_dev_starts(starts))
    torch.cuda.synchronize()
    got = host(idx[0])
    _valid_per_sequence(got, starts, w.k)
    e = ixl[0]
    kb, kd = key_bytes(e["keys"])
    rows = [0, 1, 63, 64, 129]
    ref = O.group_forward(roles, [(bits16(e["q"]), host(e["w"]), kb, kd, host(e["k_scale"])), None, None],
                          [(bits16(a["q"]), bits16(a["kv"])) for a in atl], starts, w.kv_len, w.k,
                          1.0 / math.sqrt(w.d_qk), w.d_v, rows=rows)
    np.testing.assert_array_equal(got[:, rows], ref["idx"][0])
    for l in range(3):
        err = np.abs(atl[l]["out"].float().cpu().numpy()[:, rows] - ref["O"][l]).max()
        assert err <= 2e-2, (l, err)


def test_append_keys_at_per_sequence_rows(ix):
    """Each sequence's new rows land at its own position; every other row of
    the cache is untouched."""
    rng = np.random.default_rng(21)
    B, n_new, d, cap = 4, 3, 64, 50
    seq_pos = [0, 47, 12, 30]
    k_new = rng.standard_normal((B, n_new, d)).astype(np.float32)
    cache = torch.full((B, cap, d), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((B, cap), -3.0, device="cuda")
    print(f"[varlen] append B={B} n_new={n_new} seq_pos={seq_pos}", flush=True)
    ix.ix_append_keys(torch.from_numpy(k_new).cuda(), cache, scale, seq_pos=_dev_starts(seq_pos))
    torch.cuda.synchronize()
    codes, sc = host(cache), host(scale)
    want_c, want_s = O.quantize_key_rows(k_new)
    for b, p in enumerate(seq_pos):
        np.testing.assert_array_equal(codes[b, p:p + n_new], want_c[b])
        np.testing.assert_array_equal(sc[b, p:p + n_new], want_s[b])
        keep = np.ones(cap, bool)
        keep[p:p + n_new] = False
        assert np.all(codes[b, keep] == 0x55) and np.all(sc[b, keep] == -3.0)


def test_topk_scores_long_rows_of_different_lengths(ix):
    """Per-sequence starts through the wave-local keep + merge with a
    different piece count in every row (3 to 489 pieces of 1024 scores, so
    every piece keeps 2730 down to 16 entries), normal and tied scores."""
    g = torch.Generator(device="cuda").manual_seed(7)
    L, k = 500_001, 2048
    starts = [3000, 60_000, 250_000, L - 1]
    B = len(starts)
    scores = torch.randn((B, 1, L), generator=g, device="cuda")
    scores[1] = torch.randint(-2000, 2000, (1, L), generator=g, device="cuda").float()   # ties
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    print(f"[varlen] topk_scores long rows L={L} starts={starts}", flush=True)
    ix.ix_topk_scores(scores, idx, kv_len=L, seq_q_start=_dev_starts(starts))
    torch.cuda.synchronize()
    s, got = host(scores), host(idx)
    for b in range(B):
        p = starts[b]
        np.testing.assert_array_equal(got[b, 0], O.select_topk(s[b, 0, : p + 1].astype(np.float64), k),
                                      err_msg=f"row b={b}")
