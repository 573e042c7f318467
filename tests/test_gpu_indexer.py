"""GPU parity of the full-layer indexer + top-k against the CPU oracle.

Integer-valued (exact-mode) inputs make every fp32 partial sum exact, so the
selected positions must match bit for bit; float-mode inputs are compared by
set overlap (>= 99.9%)."""
import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes, overlap, valid_idx_rows
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


def _run(ix, w, path, layer=0, inputs=None):
    if inputs is None:
        q, wt = synth.indexer_queries(w, "cuda", layer)
        keys, scale = synth.indexer_keys(w, "cuda", layer)
    else:
        q, wt, keys, scale = inputs
    idx = torch.full((w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[ix] {w.name} B={w.batch} n_q={w.n_q} kv_len={w.kv_len} k={w.k} H={w.ix_heads} "
          f"d={w.ix_dim} keys={w.key_dtype} mode={w.mode} path={path}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, path=path)
    torch.cuda.synchronize()
    return (q, wt, keys, scale), host(idx)


def _oracle(w, inputs, rows=None):
    q, wt, keys, scale = inputs
    kb, kd = key_bytes(keys)
    return O.indexer_topk(bits16(q), host(wt), kb, kd, host(scale), w.q_start, w.kv_len, w.k, rows=rows)


@pytest.mark.parametrize("path", PATHS)
def test_tiny_exact_all_rows_bit_exact(ix, path):
    w = synth.TINY_L1K
    inputs, got = _run(ix, w, path)
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
def test_exact_multi_tile_ragged(ix, path, key_dtype):
    """64 heads x 128 dims, L not a multiple of the 64-key tile, n_q not a
    multiple of the 4-row block, k small enough that the candidate buffer is
    compacted many times."""
    w = synth.L16K.with_(name="exact_l2500", n_q=2501, kv_len=2501, k=256, mode="exact",
                         key_dtype=key_dtype)
    inputs, got = _run(ix, w, path)
    valid_idx_rows(got, w.q_start, w.k)
    rows = sorted(set(range(0, 2501, 37)) | {0, 1, 255, 256, 257, 2497, 2498, 2499, 2500})
    np.testing.assert_array_equal(got[:, rows], _oracle(w, inputs, rows))


@pytest.mark.parametrize("path", PATHS)
def test_exact_k2048_fp8_with_query_offset(ix, path):
    """k = 2048 (the pages' value), fp8 keys, two sequences, and a query block
    that starts at position 3000 (chunked prefill in miniature)."""
    w = synth.CHUNK_1M.with_(name="exact_chunk", batch=2, n_q=515, q_start=3000, kv_len=3515,
                             mode="exact")
    inputs, got = _run(ix, w, path)
    valid_idx_rows(got, w.q_start, w.k)
    rows = [0, 1, 2, 3, 4, 100, 255, 256, 511, 512, 513, 514]
    np.testing.assert_array_equal(got[:, rows], _oracle(w, inputs, rows))


@pytest.mark.parametrize("path", PATHS)
def test_all_equal_scores_keep_lowest_positions(ix, path):
    """q = 0: every score is 0, so every row keeps positions 0..k-1 (ties go
    to the lower position) -- the tie-heavy worst case of the compaction."""
    w = synth.L16K.with_(name="zero_q", n_q=700, kv_len=3000, q_start=2300, k=512, mode="exact")
    q, wt = synth.indexer_queries(w, "cuda")
    keys, _ = synth.indexer_keys(w, "cuda")
    _, got = _run(ix, w, path, inputs=(torch.zeros_like(q), wt, keys, None))
    assert np.all(got == np.arange(w.k, dtype=np.int32))


@pytest.mark.parametrize("path", PATHS)
def test_increasing_scores_keep_latest_positions(ix, path):
    """score(s) = s: every key beats all earlier ones (the streaming filter's
    worst case); each row must keep its last k positions."""
    L, k = 3000, 300
    w = synth.L16K.with_(name="ramp", n_q=L, kv_len=L, k=k, ix_heads=1, ix_dim=16, mode="exact")
    s = torch.arange(L, device="cuda")
    keys = torch.zeros((1, L, 16), dtype=torch.float32, device="cuda")
    keys[0, :, 0] = torch.div(s, 16, rounding_mode="floor").float()   # <= 187: exact in bf16
    keys[0, :, 1] = (s % 16).float()
    q = torch.zeros((1, L, 1, 16), dtype=torch.float32, device="cuda")
    q[..., 0] = 16.0                                                    # q . key[s] = s
    q[..., 1] = 1.0
    inputs = (q.to(torch.bfloat16), torch.ones((1, L, 1), device="cuda"), keys.to(torch.bfloat16), None)
    assert torch.equal(inputs[2].float(), keys)
    _, got = _run(ix, w, path, inputs=inputs)
    for t in (0, 1, k - 2, k - 1, k, k + 1, 1000, L - 1):
        n = min(k, t + 1)
        assert got[0, t, :n].tolist() == list(range(t + 1 - n, t + 1))


@pytest.mark.parametrize("increasing", [True, False])
def test_long_ramp_rows_on_the_few_rows_path(ix, increasing):
    """Few long rows on the materialised path (score kernel with the top-k's
    wave-local keep, then the merge): with score(s) = s every row's k best
    sit in its last waves' pieces, with score(s) = L-1-s in its first ones,
    so pieces drop winners and the merge must fall back to the whole-row
    select.  Scores are exact: q = (4096, 64, 1) and the key holds the base-64
    digits of s (or of L-1-s), all exact in bf16."""
    L, k, n_q = 150_001, 2048, 3
    w = synth.L16K.with_(name="long_ramp", batch=2, n_q=n_q, q_start=L - n_q, kv_len=L, k=k, ix_heads=1,
                         ix_dim=16, mode="exact")
    s = torch.arange(L, device="cuda")
    v = s if increasing else (L - 1 - s)
    keys = torch.zeros((2, L, 16), dtype=torch.float32, device="cuda")
    keys[:, :, 0] = torch.div(v, 4096, rounding_mode="floor").float()
    keys[:, :, 1] = (torch.div(v, 64, rounding_mode="floor") % 64).float()
    keys[:, :, 2] = (v % 64).float()
    q = torch.zeros((2, n_q, 1, 16), dtype=torch.float32, device="cuda")
    q[..., 0], q[..., 1], q[..., 2] = 4096.0, 64.0, 1.0
    inputs = (q.to(torch.bfloat16), torch.ones((2, n_q, 1), device="cuda"), keys.to(torch.bfloat16), None)
    assert torch.equal(inputs[2].float(), keys)
    _, got = _run(ix, w, 2, inputs=inputs)
    for b in range(2):
        for t in range(n_q):
            p = w.q_start + t
            want = list(range(p + 1 - k, p + 1)) if increasing else list(range(k))
            assert got[b, t].tolist() == want, f"b={b} t={t}"


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kv_len", [327_680, 400_001])
def test_exact_few_long_rows_both_score_kernel_modes(ix, key_dtype, kv_len):
    """Few long rows on the materialised path at the edge of the score
    kernel's two modes: rows of up to 512 waves' spans (327,680 keys) keep
    each wave's best for the one-pass merge (here 16 slots per wave, the
    fewest it allows), longer rows get per-wave score ranges for the
    five-pass select.  Integer-valued inputs: bit-exact against the oracle."""
    w = synth.DECODE_B32.with_(name=f"exact_long_{kv_len}", batch=2, n_q=2, q_start=kv_len - 2, kv_len=kv_len,
                               ix_heads=4, ix_dim=32, key_dtype=key_dtype, mode="exact", decode_steps=0,
                               kv_cap=0)
    inputs, got = _run(ix, w, 2)
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs))


@pytest.mark.parametrize("path", PATHS)
def test_fp8_every_code_orders_like_the_oracle(ix, path):
    """One key per e4m3fn code (NaN codes excluded), scored by a unit query:
    the selection at several k must match the oracle's decode of the codes."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    L = len(codes)
    w = synth.CHUNK_1M.with_(name="codes", n_q=4, q_start=L - 4, kv_len=L, ix_heads=1, ix_dim=16,
                             k=64, mode="exact")
    keys = torch.zeros((1, L, 16), dtype=torch.uint8, device="cuda")
    keys[0, :, 0] = torch.from_numpy(codes).cuda()
    scale = torch.ones((1, L), dtype=torch.float32, device="cuda")
    q = torch.zeros((1, 4, 1, 16), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = 1.0
    wt = torch.tensor([1.0, -1.0, 2.0, -0.5], device="cuda").view(1, 4, 1)
    for k in (1, 7, 64, 200):
        wk = w.with_(k=k)
        inputs, got = _run(ix, wk, path, inputs=(q, wt, keys, scale))
        np.testing.assert_array_equal(got, _oracle(wk, inputs))


@pytest.mark.parametrize("path", PATHS)
def test_float_mode_overlap(ix, path):
    """N(0, 1/sqrt(d)) queries, N(0,1) weights: fp32 GPU sums vs float64
    oracle may split near-ties, so compare sets: >= 99.9% overall."""
    w = synth.L16K.with_(name="float_l4096", n_q=4096, kv_len=4096, k=512)
    inputs, got = _run(ix, w, path)
    valid_idx_rows(got, w.q_start, w.k)
    rows = sorted(set(range(0, 4096, 61)) | {511, 512, 513, 4095})
    ov, worst = overlap(got[:, rows], _oracle(w, inputs, rows))
    print(f"overlap {ov:.6f} worst row {worst:.6f}")
    assert ov >= 0.999


def test_fused_and_materialised_paths_agree(ix):
    w = synth.L16K.with_(name="float_paths", n_q=1500, kv_len=1500, k=1024, key_dtype="fp8")
    inputs, a = _run(ix, w, 1)
    _, b = _run(ix, w, 2, inputs=inputs)
    ov, _ = overlap(a, b)
    assert ov >= 0.9999


def test_topk_scores_entry_point(ix):
    """ix_topk_scores on caller-provided rows with heavy ties."""
    g = torch.Generator(device="cuda").manual_seed(5)
    B, n_q, L, k = 2, 6, 5000, 700
    scores = torch.randint(-40, 40, (B, n_q, L), generator=g, device="cuda").float()
    scores[0, 0] = -0.0
    idx = torch.empty((B, n_q, k), dtype=torch.int32, device="cuda")
    q_start = L - n_q
    ix.ix_topk_scores(scores, idx, q_start=q_start, kv_len=L)
    torch.cuda.synchronize()
    s = host(scores)
    got = host(idx)
    for b in range(B):
        for t in range(n_q):
            p = q_start + t
            np.testing.assert_array_equal(got[b, t], O.select_topk(s[b, t, : p + 1].astype(np.float64), k))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
def test_exact_spare_cache_rows_and_batch(ix, path, key_dtype):
    """Two sequences whose key caches hold spare rows past kv_len (kv_cap >
    kv_len) and a query block at q_start > 0.  The spare rows are poisoned with
    the largest key values, so reading keys with the wrong sequence stride, or
    past kv_len, would change the selection."""
    w = synth.L16K.with_(name="exact_cap", batch=2, n_q=300, q_start=900, kv_len=1200, kv_cap=1300,
                         k=256, mode="exact", key_dtype=key_dtype)
    q, wt = synth.indexer_queries(w, "cuda", 0)
    keys, scale = synth.indexer_keys(w, "cuda", 0)
    poison = torch.full_like(keys[:, w.kv_len:], 0)
    if key_dtype == "bf16":
        poison = torch.full(poison.shape, 8.0, dtype=torch.bfloat16, device="cuda")
    else:
        poison = torch.full(poison.shape, 8.0, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8)
    keys[:, w.kv_len:] = poison
    inputs, got = _run(ix, w, path, inputs=(q, wt, keys, scale))
    valid_idx_rows(got, w.q_start, w.k)
    rows = [0, 1, 150, 298, 299]
    np.testing.assert_array_equal(got[:, rows], _oracle(w, inputs, rows))
