"""Row top-k over caller-provided fp32 scores (ix_topk_scores), on every
select path: for few long rows the wave-local keep over pieces of 1024
positions + per-row merge (rows of up to 512 pieces, with its whole-row
fallback when a piece dropped an entry that could rank among the k best, as
on monotone ramps, or too few were kept) and the five-pass chunked select for
longer rows (with its fallback when the k-th best sits in an over-full value
bin); the single-workgroup select for many rows, unaligned row strides and
rows short enough to keep every position.  Compared with the oracle's stable
sort, element for element."""
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


def _check(ix, scores, k, q_start, kv_len, rows=None):
    B, n_q, _ = scores.shape
    idx = torch.full((B, n_q, k), -7, dtype=torch.int32, device="cuda")
    print(f"[topk] B={B} n_q={n_q} ld={scores.shape[2]} kv_len={kv_len} q_start={q_start} k={k}", flush=True)
    ix.ix_topk_scores(scores, idx, q_start=q_start, kv_len=kv_len)
    torch.cuda.synchronize()
    s, got = host(scores), host(idx)
    for b in range(B):
        for t in (range(n_q) if rows is None else rows):
            p = q_start + t
            np.testing.assert_array_equal(got[b, t], O.select_topk(s[b, t, :p + 1].astype(np.float64), k),
                                          err_msg=f"row b={b} t={t}")


def test_chunked_long_rows_normal(ix):
    g = torch.Generator(device="cuda").manual_seed(11)
    L = 200_003
    scores = torch.randn((4, 1, L), generator=g, device="cuda")
    _check(ix, scores, 2048, L - 1, L)


def test_chunked_long_rows_integer_ties(ix):
    g = torch.Generator(device="cuda").manual_seed(12)
    L = 70_000
    scores = torch.randint(-300, 300, (3, 2, L), generator=g, device="cuda").float()
    _check(ix, scores, 2048, L - 2, L)


def test_chunked_unaligned_stride(ix):
    g = torch.Generator(device="cuda").manual_seed(13)
    L = 30_001
    base = torch.randn((2, 1, L + 1), generator=g, device="cuda")
    _check(ix, base, 1000, L - 1, L)       # ld = L + 1: rows not 16-byte aligned


def test_chunked_fallback_flat_rows(ix):
    """Every score equal, or one outlier stretching the range: the k-th best
    shares its bin with far more than the candidate capacity."""
    L = 40_000
    flat = torch.full((1, 1, L), 3.25, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(14)
    outlier = torch.randn((1, 1, L), generator=g, device="cuda")
    outlier[0, 0, 123] = 1e30
    signed_zero = torch.zeros((1, 1, L), device="cuda")
    signed_zero[0, 0, ::3] = -0.0
    for s in (flat, outlier, signed_zero):
        _check(ix, s, 2048, L - 1, L)


def test_chunked_monotone_ramps_fall_back(ix):
    """The k best all sit in the last (increasing) or first (decreasing)
    chunk: that chunk keeps only 8192 / chunks of them, so its dropped keys
    outrank the merged k-th best and the row takes the whole-row select."""
    L = 200_001
    up = torch.arange(L, device="cuda", dtype=torch.float32).reshape(1, 1, L)
    down = torch.flip(up, dims=[2]).contiguous()
    _check(ix, torch.cat([up, down], dim=0), 2048, L - 1, L)


def test_chunked_local_path_at_its_longest_rows(ix):
    """512 pieces of 1024 (the longest rows of the keep + merge passes): each
    piece keeps at most 16 entries."""
    g = torch.Generator(device="cuda").manual_seed(17)
    L = 512 * 1024
    scores = torch.randn((2, 1, L), generator=g, device="cuda")
    _check(ix, scores, 2048, L - 1, L)


def test_chunked_five_pass_path_past_512_pieces(ix):
    """Rows of more than 512 pieces use the range / histogram / select /
    collect / finish passes (one row just past the limit, one past 1M)."""
    g = torch.Generator(device="cuda").manual_seed(18)
    for L in (512 * 1024 + 1, 128 * 8192 + 5001):
        scores = torch.randn((2, 1, L), generator=g, device="cuda")
        ties = torch.randint(-50, 50, (1, 1, L), generator=g, device="cuda").float()
        _check(ix, torch.cat([scores, ties], dim=0), 2048, L - 1, L)


@pytest.mark.parametrize("L", [2049, 5000, 8192, 9000])
def test_local_pieces_that_keep_everything(ix, L):
    """Rows of at most 8 pieces give each piece at least 1024 slots, so a
    full piece keeps all its scores (the row's k-th best is then found by the
    merge alone); 9000 positions is the first row past that."""
    g = torch.Generator(device="cuda").manual_seed(19)
    scores = torch.randn((3, 1, L), generator=g, device="cuda")
    _check(ix, scores, 2048, L - 1, L)


def test_local_signed_zero_ties_through_the_merge(ix):
    """Rare 2.0s, many zeros of both signs and negatives elsewhere: every
    piece keeps its 2.0s and zeros, the row's k-th best is a zero, and the
    merge keeps the earliest zeros of either sign (-0 and +0 rank equal)."""
    g = torch.Generator(device="cuda").manual_seed(20)
    L = 40_000
    u = torch.rand((2, 1, L), generator=g, device="cuda")
    s = torch.where(u < 0.001, torch.full_like(u, 2.0),
                    torch.where(u < 0.05, torch.zeros_like(u),
                                torch.where(u < 0.1, torch.full_like(u, -0.0), -1.0 - u)))
    assert int((s == 2.0).sum()) < 2 * 256 and int((s == 0).sum()) > 2 * 256
    _check(ix, s, 256, L - 1, L)


@pytest.mark.parametrize("k", [1, 7, 2047])
def test_local_path_small_and_odd_k(ix, k):
    """The keep + merge at k = 1 (the row's first maximum), a small odd k and
    k = 2047, on normal rows and on integer rows where the k-th best is tied
    many times over."""
    g = torch.Generator(device="cuda").manual_seed(21 + k)
    L = 100_003
    normal = torch.randn((2, 1, L), generator=g, device="cuda")
    ties = torch.randint(-40, 40, (2, 1, L), generator=g, device="cuda").float()
    _check(ix, torch.cat([normal, ties], dim=0), k, L - 1, L)


def test_chunked_ragged_rows_with_short_prefix(ix):
    """Rows 0.. of a prefill chunk: the first rows keep every position."""
    g = torch.Generator(device="cuda").manual_seed(15)
    n_q = 600
    scores = torch.randn((1, n_q, n_q), generator=g, device="cuda")
    _check(ix, scores, 256, 0, n_q)


def test_single_workgroup_many_rows(ix):
    g = torch.Generator(device="cuda").manual_seed(16)
    n_q, L = 1100, 3000
    scores = torch.randn((1, n_q, L), generator=g, device="cuda")
    _check(ix, scores, 512, L - n_q, L, rows=[0, 1, 517, 1099])
