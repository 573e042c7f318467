"""GPU parity of ix_indexer_project (the indexer's q_I and head weights from
hidden states, IndexCache notes, section 1) against the CPU oracle's
indexer_project.

Exact mode (integer inputs in [-8, 8]): every fp32 partial sum is an integer
below 2^24, so q_I (rounded to bf16 from an exact value) matches bit for bit
and w exactly.  Float mode: the GPU accumulates in fp32 in its own order, so
q_I may differ from the oracle's bf16(exact) by one unit in the last place
where the exact value sits within rounding error of a midpoint (a small
fraction of elements); w agrees within fp32 accumulation error."""
import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _inputs(rows, d_in, heads, dim, mode, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    n = heads * dim + heads
    if mode == "exact":
        x = torch.randint(-8, 9, (rows, d_in), generator=g, device="cuda", dtype=torch.int32).to(torch.bfloat16)
        w = torch.randint(-8, 9, (n, d_in), generator=g, device="cuda", dtype=torch.int32).to(torch.bfloat16)
    else:
        x = torch.randn((rows, d_in), generator=g, device="cuda").to(torch.bfloat16)
        w = (torch.randn((n, d_in), generator=g, device="cuda") / d_in ** 0.5).to(torch.bfloat16)
    return x, w


def _run(ix, x, w, heads, dim):
    rows = x.shape[0]
    q = torch.full((rows, heads, dim), 7, dtype=torch.bfloat16, device="cuda")
    wo = torch.full((rows, heads), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[project] rows={rows} d_in={x.shape[1]} heads={heads} dim={dim}", flush=True)
    ix.ix_indexer_project(x, w, q, wo, heads=heads, dim=dim)
    torch.cuda.synchronize()
    return bits16(q), host(wo)


@pytest.mark.parametrize("rows,d_in,heads,dim", [
    (300, 512, 64, 128),      # 256-row tiles: a ragged row tile, 8256 columns (32.25 tiles)
    (129, 192, 3, 40),        # one row past the few-rows limit, odd head count
    (1, 64, 5, 16),           # 64-row tiles from here on: a single row, a single K step
    (100, 320, 3, 40),        # two ragged row tiles, odd K steps, a ragged column tile
    (128, 128, 2, 64),        # the few-rows limit itself
    (32, 6144, 64, 128),      # a decode batch at the model's width
])
def test_exact_bit_exact(ix, rows, d_in, heads, dim):
    """Both tile shapes (256 x 256 above 128 rows, 64 x 64 up to it), ragged
    row and column tiles, a single row, single and odd K step counts, odd
    head counts, and a decode batch at full width."""
    x, w = _inputs(rows, d_in, heads, dim, "exact", rows)
    q, wo = _run(ix, x, w, heads, dim)
    q_ref, w_ref = O.indexer_project(bits16(x), bits16(w), heads, dim)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(wo.astype(np.float64), w_ref)


def test_float_within_one_ulp(ix):
    """Each q_I element within one bf16 unit of the oracle's value (or within
    twice the fp32 accumulation bound, for outputs near zero), differing in a
    small fraction of elements; w within the accumulation bound."""
    rows, d_in, heads, dim = 257, 1024, 64, 128
    x, w = _inputs(rows, d_in, heads, dim, "float", 3)
    q, wo = _run(ix, x, w, heads, dim)
    q_ref, w_ref = O.indexer_project(bits16(x), bits16(w), heads, dim)
    X, W = O.decode_bf16(bits16(x)), O.decode_bf16(bits16(w))
    bound = 1e-5 * (np.abs(X) @ np.abs(W).T)               # fp32 accumulation, generous
    got, ref = O.decode_bf16(q).reshape(rows, -1), O.decode_bf16(q_ref).reshape(rows, -1)
    ulp = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    diff = np.abs(got - ref)
    assert np.all(diff <= np.maximum(ulp, 2 * bound[:, : heads * dim]))
    assert np.mean(diff != 0) <= 5e-3, np.mean(diff != 0)
    assert np.all(np.abs(wo - w_ref) <= bound[:, heads * dim:])


def test_full_size_sampled_rows(ix):
    """The shape the bench times: 131,072 rows of width 6144 into 64 heads x
    128 plus 64 weights; 24 rows (first, last and seeded) against the
    oracle, in exact mode so they must match bit for bit."""
    rows, d_in, heads, dim = 131072, 6144, 64, 128
    x, w = _inputs(rows, d_in, heads, dim, "exact", 17)
    q, wo = _run(ix, x, w, heads, dim)
    rng = np.random.default_rng(0)
    sample = sorted({0, rows - 1, *rng.integers(0, rows, 22).tolist()})
    xb = bits16(x[sample])
    q_ref, w_ref = O.indexer_project(xb, bits16(w), heads, dim)
    np.testing.assert_array_equal(q[sample], q_ref)
    np.testing.assert_array_equal(wo[sample].astype(np.float64), w_ref)


def test_zero_rows_and_bad_shapes(ix):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2 * 16 + 2, 64), dtype=torch.bfloat16, device="cuda")
    ix.ix_indexer_project(x, w, torch.empty((0, 2, 16), dtype=torch.bfloat16, device="cuda"),
                          torch.empty((0, 2), device="cuda"), heads=2, dim=16)
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2 * 16 + 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ix.IxError):
        ix.ix_indexer_project(x, w, torch.empty((4, 2, 16), dtype=torch.bfloat16, device="cuda"),
                              torch.empty((4, 2), device="cuda"), heads=2, dim=16)
