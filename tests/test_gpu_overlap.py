"""Per-row overlap of two index buffers (ix_index_overlap) against the
oracle's set intersection, bit for bit."""
import numpy as np
import pytest
import torch

from helpers import ensure_lib, host
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


def _rows(rng, n_rows, k, universe, sizes):
    out = np.full((n_rows, k), -1, dtype=np.int32)
    for r in range(n_rows):
        n = sizes[r]
        out[r, :n] = np.sort(rng.choice(universe, size=n, replace=False))
    return out


@pytest.mark.parametrize("k", [2048, 1, 3, 100, 1000, 1001, 2044])
def test_constructed_rows_with_known_overlap(ix, k):
    """b shares a prescribed number of positions with a (the rest drawn from
    outside a), with padded rows, empty rows and full rows; k = 2048, 2044
    and 1000 take the kernel's 16-byte loads (2044 and 1000 with lanes past
    the row's end), the others its 4-byte ones."""
    rng = np.random.default_rng(7 + k)
    B, n_q = 2, 150
    rows = B * n_q
    sizes = rng.integers(0, k + 1, size=rows)
    sizes[:3] = [0, k, min(1, k)]
    a = _rows(rng, rows, k, 100_000, sizes)
    b = np.full_like(a, -1)
    want = np.zeros(rows, dtype=np.int64)
    for r in range(rows):
        va = a[r, :sizes[r]]
        common = rng.integers(0, sizes[r] + 1)
        keep = rng.choice(va, size=common, replace=False) if common else np.zeros(0, np.int32)
        extra_n = rng.integers(0, k - common + 1)
        extra = rng.choice(np.arange(100_000, 300_000), size=extra_n, replace=False)
        vb = np.sort(np.concatenate([keep, extra]).astype(np.int32))
        b[r, :vb.shape[0]] = vb
        want[r] = common
    ta = torch.from_numpy(a.reshape(B, n_q, k)).cuda()
    tb = torch.from_numpy(b.reshape(B, n_q, k)).cuda()
    print(f"[overlap] B={B} n_q={n_q} k={k}", flush=True)
    got = host(ix.ix_index_overlap(ta, tb)).reshape(-1)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(got, O.index_overlap(a, b))
    np.testing.assert_array_equal(host(ix.ix_index_overlap(ta, ta)).reshape(-1), sizes)


def test_two_indexer_layers(ix):
    """Index buffers the indexer itself wrote for two different layers of one
    prefill chunk (rows with fewer than k candidates padded with -1)."""
    w = synth.L16K.with_(name="overlap_layers", n_q=1500, kv_len=1500, k=512)
    bufs = []
    for layer in (0, 4):
        q, wt = synth.indexer_queries(w, "cuda", layer)
        keys, scale = synth.indexer_keys(w, "cuda", layer)
        idx = torch.empty((1, w.n_q, w.k), dtype=torch.int32, device="cuda")
        ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=0, kv_len=w.kv_len)
        bufs.append(idx)
    got = host(ix.ix_index_overlap(bufs[0], bufs[1]))
    np.testing.assert_array_equal(got, O.index_overlap(host(bufs[0]), host(bufs[1])))
    # rows with p + 1 <= k keep every position in both layers
    np.testing.assert_array_equal(got[0, :w.k], np.arange(1, w.k + 1))
