"""New indexer keys into the fp8 cache (ix_append_keys) against the oracle's
quantizer: codes and scales bit for bit, other cache rows untouched."""
import numpy as np
import pytest
import torch

from helpers import ensure_lib, host
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _append(ix, k_new, cap, pos):
    B, n_new, d = k_new.shape
    cache = torch.full((B, cap, d), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.full((B, cap), -3.0, device="cuda")
    print(f"[append] B={B} n_new={n_new} d={d} cap={cap} pos={pos}", flush=True)
    ix.ix_append_keys(torch.from_numpy(k_new).cuda(), cache, scale, pos)
    torch.cuda.synchronize()
    return host(cache), host(scale)


def _check(ix, k_new, cap, pos):
    codes, sc = _append(ix, k_new, cap, pos)
    want_c, want_s = O.quantize_key_rows(k_new)
    n = k_new.shape[1]
    np.testing.assert_array_equal(codes[:, pos:pos + n], want_c)
    np.testing.assert_array_equal(sc[:, pos:pos + n], want_s)
    assert np.all(codes[:, :pos] == 0x55) and np.all(codes[:, pos + n:] == 0x55)
    assert np.all(sc[:, :pos] == -3.0) and np.all(sc[:, pos + n:] == -3.0)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_random_rows_all_scales(ix, d):
    rng = np.random.default_rng(d)
    k = rng.standard_normal((3, 5, d)).astype(np.float32)
    k *= np.array([1e-3, 1.0, 37.5, 1e4, 0.25], dtype=np.float32)[None, :, None]
    _check(ix, k, 40, 17)


def test_zero_rows_lone_values_and_signed_zeros(ix):
    k = np.zeros((1, 4, 32), dtype=np.float32)
    k[0, 1, 5] = -2.5                               # one nonzero: it maps to -448, the rest to +0
    k[0, 2, :] = -0.0                               # all negative zeros: scale 1, codes +0
    k[0, 3, ::2] = 1e-30                            # tiny values next to a large one
    k[0, 3, 1] = 3.0e4
    _check(ix, k, 8, 2)


def test_exact_rounding_ties(ix):
    """A row whose largest magnitude is 448 (scale 1) and whose other entries
    sit exactly halfway between neighbouring e4m3fn values: every one is a
    tie that must go to the even code, as in the oracle."""
    vals = O.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    fin = np.sort(np.unique(vals[~np.isnan(vals)]))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    mids = mids[np.abs(mids) < 448]
    row = np.concatenate([[448.0], mids]).astype(np.float32)
    d = 128
    rows = []
    for start in range(0, row.shape[0], d - 1):
        r = np.concatenate([[448.0], row[1 + start:1 + start + d - 1]])
        r = np.pad(r, (0, d - r.shape[0]))
        rows.append(r)
    k = np.stack(rows)[None].astype(np.float32)
    _check(ix, k, k.shape[1] + 3, 3)
