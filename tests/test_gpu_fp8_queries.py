"""GPU parity of the fp8-query indexer (queries as e4m3fn codes times one fp32
scale per (row, head); IndexCache notes, section 1: an FP8 indexer) against
the CPU oracle.

Two kernel forms are covered: with fp8 keys and d in {64, 128} the fused
kernel multiplies the codes on the fp8 MFMA and reads the key cache in place;
otherwise (bf16 keys, other d, the materialised path) the codes are widened
to bf16.  Integer-valued inputs with power-of-two scales keep every partial
sum exact on both forms, so positions must match bit for bit; float-mode
inputs are compared by set overlap."""
import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes, overlap, valid_idx_rows
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


def _inputs(w, layer=0):
    q, qs, wt = synth.indexer_queries_fp8(w, "cuda", layer)
    keys, scale = synth.indexer_keys(w, "cuda", layer)
    return q, qs, wt, keys, scale


def _run(ix, w, path, inputs):
    q, qs, wt, keys, scale = inputs
    idx = torch.full((w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[ix8] {w.name} B={w.batch} n_q={w.n_q} q_start={w.q_start} kv_len={w.kv_len} cap={w.cap} "
          f"k={w.k} H={w.ix_heads} d={w.ix_dim} keys={w.key_dtype} mode={w.mode} path={path}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, path=path,
                       q_scale=qs)
    torch.cuda.synchronize()
    return host(idx)


def _oracle(w, inputs, rows=None):
    q, qs, wt, keys, scale = inputs
    kb, kd = key_bytes(keys)
    return O.indexer_topk(host(q), host(wt), kb, kd, host(scale), w.q_start, w.kv_len, w.k, rows=rows,
                          q_scale=host(qs))


BASE = synth.L16K.with_(name="fp8q_exact", batch=2, n_q=301, q_start=700, kv_len=1001, k=256,
                        key_dtype="fp8", mode="exact")


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("key_dtype,heads,dim", [
    ("fp8", 64, 128),     # fp8 MFMA form, two head tiles
    ("fp8", 40, 64),      # fp8 MFMA form, d = 64, partial second head tile
    ("fp8", 3, 128),      # fp8 MFMA form, one head tile
    ("fp8", 17, 64),
    ("fp8", 5, 32),       # widened form (no fp8 MFMA for d = 32)
    ("fp8", 7, 16),       # widened form, the narrowest key
    ("bf16", 64, 128),    # widened form (bf16 keys)
])
def test_exact_bit_exact(ix, path, key_dtype, heads, dim):
    """Ragged tiles (L not a multiple of 64), a partial last row block, two
    sequences, a chunk that starts mid-way: positions bit for bit."""
    w = BASE.with_(name=f"fp8q_exact_{key_dtype}_{heads}x{dim}", key_dtype=key_dtype, ix_heads=heads,
                   ix_dim=dim)
    inputs = _inputs(w)
    got = _run(ix, w, path, inputs)
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs))


@pytest.mark.parametrize("key_dtype", ["fp8", "bf16"])
@pytest.mark.parametrize("heads,dim", [(64, 48), (40, 80), (33, 112)])
def test_materialised_widths(ix, key_dtype, heads, dim):
    """Widths the fused kernel does not take (the materialised path widens
    the codes for every multiple of 16): positions bit for bit."""
    w = BASE.with_(name=f"fp8q_width_{key_dtype}_{heads}x{dim}", batch=1, key_dtype=key_dtype, ix_heads=heads,
                   ix_dim=dim)
    inputs = _inputs(w)
    got = _run(ix, w, 0, inputs)
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs))


@pytest.mark.parametrize("dim", [64, 128])
@pytest.mark.parametrize("spare", [0, 5, 70])
def test_cache_read_in_place_spare_rows(ix, dim, spare):
    """The fp8 MFMA form reads the key cache itself: spare rows past kv_len
    hold NaN codes and NaN scales and must not matter; with no spare rows the
    last tile runs off the end of the cache (those rows read as zeros)."""
    w = BASE.with_(name=f"fp8q_spare_{dim}_{spare}", batch=1, n_q=130, q_start=871, kv_len=1001,
                   kv_cap=1001 + spare, ix_dim=dim, k=300)
    q, qs, wt, keys, scale = _inputs(w)
    keys[:, w.kv_len:] = 0x7F
    scale[:, w.kv_len:] = float("nan")
    got = _run(ix, w, 1, (q, qs, wt, keys, scale))
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, (q, qs, wt, keys, scale)))


@pytest.mark.parametrize("path", [1, 2])
def test_float_mode_overlap(ix, path):
    """amax-scaled fp8 queries and keys, N(0, 1) weights: the GPU's fp32 (and,
    in the fused fp8 MFMA form, the matrix core's narrower internal) sums
    against the float64 oracle over the same codes may split near-ties, so
    compare sets."""
    w = synth.L16K.with_(name="fp8q_float_l4096", n_q=4096, kv_len=4096, k=512, key_dtype="fp8")
    inputs = _inputs(w)
    got = _run(ix, w, path, inputs)
    valid_idx_rows(got, w.q_start, w.k)
    rows = sorted(set(range(0, 4096, 61)) | {511, 512, 513, 4095})
    ov, worst = overlap(got[:, rows], _oracle(w, inputs, rows))
    print(f"overlap {ov:.6f} worst row {worst:.6f}")
    assert ov >= 0.999


def test_fp8_and_widened_forms_agree(ix):
    """The fused fp8 MFMA form against the materialised path (codes widened
    to bf16, exact products, fp32 sums) on float inputs."""
    w = synth.L16K.with_(name="fp8q_forms", n_q=1500, kv_len=1500, k=1024, key_dtype="fp8")
    inputs = _inputs(w)
    a = _run(ix, w, 1, inputs)
    b = _run(ix, w, 2, inputs)
    ov, _ = overlap(a, b)
    print(f"overlap {ov:.6f}")
    assert ov >= 0.999


def test_power_of_two_scales_equal_the_bf16_query_run(ix):
    """Codes times power-of-two scales are exact bf16 values: the same
    problem posed with bf16 queries selects the same positions."""
    w = BASE.with_(name="fp8q_vs_bf16", batch=1)
    q, qs, wt, keys, scale = _inputs(w)
    q16 = (q.view(torch.float8_e4m3fn).float() * qs[..., None]).to(torch.bfloat16)
    got8 = _run(ix, w, 1, (q, qs, wt, keys, scale))
    idx16 = torch.full_like(torch.from_numpy(got8).cuda(), -7)
    ix.ix_indexer_topk(q16, wt, keys, idx16, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, path=1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got8, host(idx16))


@pytest.mark.parametrize("dim", [64, 128, 32])
def test_argmax_exact(ix, dim):
    """The top-1 entry point on fp8 queries: position (ties -> lower) and
    score bit for bit."""
    w = BASE.with_(name=f"fp8q_argmax_{dim}", batch=1, n_q=257, ix_dim=dim, ix_heads=33)
    q, qs, wt, keys, scale = _inputs(w)
    pos = torch.full((1, w.n_q), -7, dtype=torch.int32, device="cuda")
    score = torch.full((1, w.n_q), float("nan"), device="cuda")
    print(f"[ix8 argmax] d={dim} n_q={w.n_q}", flush=True)
    ix.ix_indexer_argmax(q, wt, keys, pos, score, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len,
                         q_scale=qs)
    torch.cuda.synchronize()
    pos, score = host(pos), host(score)
    kb, kd = key_bytes(keys)
    kmat = O.key_matrix(kb[0, : w.kv_len], kd, host(scale)[0, : w.kv_len])
    qh, qsh, wh = host(q)[0], host(qs)[0], host(wt)[0]
    for t in range(0, w.n_q, 4):
        n = w.q_start + t + 1
        s = O.indexer_scores(O.query_matrix(qh[t], qsh[t]), np.asarray(wh[t], np.float64), kmat[:n])
        p_ref = int(O.select_topk(s, 1)[0])
        assert pos[0, t] == p_ref, t
        assert score[0, t] == s[p_ref], t


def test_group_slot_equals_standalone_call(ix):
    """A full layer with fp8 queries inside ix_group_forward fills its slot
    exactly as the standalone call does."""
    w = synth.TINY_L1K.with_(name="fp8q_group", key_dtype="fp8", ix_heads=64, ix_dim=128, mode="exact")
    q, qs, wt, keys, scale = _inputs(w)
    ixl = [dict(q=q, w=wt, keys=keys, k_scale=scale, q_scale=qs), None, None, None]
    atl = []
    for l in range(4):
        atl.append(dict(q=synth.attn_queries(w, "cuda", l), kv=synth.latent_kv(w, "cuda", l),
                        out=torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16,
                                        device="cuda"),
                        lse=torch.empty((w.batch, w.n_q, w.q_heads), device="cuda")))
    idx = torch.full((1, w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    ix.ix_group_forward(ixl, atl, 1, idx, q_start=w.q_start, kv_len=w.kv_len)
    solo = torch.full_like(idx[0], -7)
    ix.ix_indexer_topk(q, wt, keys, solo, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, q_scale=qs)
    torch.cuda.synchronize()
    assert torch.equal(solo, idx[0])
    np.testing.assert_array_equal(host(idx[0]), _oracle(w, (q, qs, wt, keys, scale)))


def test_binding_rejects_mismatched_query_forms(ix):
    w = BASE.with_(name="fp8q_bad", batch=1, n_q=8, q_start=0, kv_len=8, k=4)
    q, qs, wt, keys, scale = _inputs(w)
    idx = torch.empty((1, 8, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(Exception):
        ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=0, kv_len=8)              # no q_scale
    q16 = torch.zeros(q.shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(Exception):
        ix.ix_indexer_topk(q16, wt, keys, idx, k_scale=scale, q_start=0, kv_len=8, q_scale=qs)


def _planted_rows(dim, n=333, seed=5):
    """bf16 query rows: seeded N(0,1) rows whose scales span 1e-3..1e3, then
    an all-zero row, a constant row (every code 448), a row whose small
    values land on subnormal codes and round to +0 / -0, and a row with one
    huge and otherwise tiny values."""
    g = torch.Generator(device="cpu").manual_seed(seed + dim)
    q = torch.randn((n, dim), generator=g) * torch.logspace(-3, 3, n).unsqueeze(1)
    q[0] = 0.0
    q[1] = 1.5
    q[2] = torch.tensor([1.0, 2e-5, -2e-5, 1e-6, -1e-6, 3e-5, -7e-6, 0.0] * (dim // 8))
    q[3] = -1e-7
    q[3, 5] = 3.0e4
    return q.to(torch.bfloat16)


@pytest.mark.parametrize("dim", [16, 48, 64, 128])
def test_quantize_queries_bit_exact(ix, dim):
    """ix_quantize_queries against the oracle's key-row quantiser applied to
    every row of the same bf16 values: codes and scales bit for bit."""
    q = _planted_rows(dim)
    print(f"[quantize] dim={dim} rows={q.shape[0]}", flush=True)
    codes, scale = ix.ix_quantize_queries(q.cuda())
    torch.cuda.synchronize()
    ref_c, ref_s = O.quantize_key_rows(O.decode_bf16(bits16(q)))
    np.testing.assert_array_equal(host(codes), ref_c)
    np.testing.assert_array_equal(host(scale).view(np.uint32), ref_s.astype(np.float32).view(np.uint32))


def test_quantize_queries_shapes(ix):
    """A [B, n_q, H, d] query tensor maps to [B, n_q, H] scales; zero rows do
    nothing; sizes the kernel does not take are refused."""
    q = _planted_rows(64, n=2 * 3 * 5).view(2, 3, 5, 64).cuda()
    codes, scale = ix.ix_quantize_queries(q)
    torch.cuda.synchronize()
    assert codes.shape == (2, 3, 5, 64) and scale.shape == (2, 3, 5)
    ref_c, ref_s = O.quantize_key_rows(O.decode_bf16(bits16(q)))
    np.testing.assert_array_equal(host(codes), ref_c)
    np.testing.assert_array_equal(host(scale), ref_s)
    ix.ix_quantize_queries(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(Exception):
        ix.ix_quantize_queries(torch.zeros((4, 40), dtype=torch.bfloat16, device="cuda"))


def test_projected_queries_through_the_fp8_indexer(ix):
    """Hidden rows -> ix_indexer_project (bf16 q) -> ix_quantize_queries ->
    fp8-query indexer, against the oracle's projection, quantiser and
    indexer: the codes and scales bit for bit (integer hidden rows and
    weights make the projection exact on both sides), then the selected sets
    (the non-power-of-two scales make the scores inexact) by overlap."""
    w = synth.L16K.with_(name="fp8q_projected", n_q=700, kv_len=700, k=256, key_dtype="fp8", mode="exact")
    x, wp = synth.projection_inputs(w, "cuda", d_in=256)
    keys, kscale = synth.indexer_keys(w, "cuda", 0)
    H, d = w.ix_heads, w.ix_dim
    q16 = torch.empty((1, w.n_q, H, d), dtype=torch.bfloat16, device="cuda")
    wt = torch.empty((1, w.n_q, H), dtype=torch.float32, device="cuda")
    print(f"[projected fp8 indexer] n_q={w.n_q} H={H} d={d}", flush=True)
    ix.ix_indexer_project(x.view(1, w.n_q, -1), wp, q16, wt, heads=H, dim=d)
    codes, qs = ix.ix_quantize_queries(q16)
    idx = torch.full((1, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    ix.ix_indexer_topk(codes, wt, keys, idx, k_scale=kscale, q_start=0, kv_len=w.kv_len, q_scale=qs)
    torch.cuda.synchronize()
    q_ref, w_ref = O.indexer_project(bits16(x), bits16(wp), H, d)
    c_ref, s_ref = O.quantize_key_rows(O.decode_bf16(q_ref))
    np.testing.assert_array_equal(host(codes).reshape(c_ref.shape), c_ref)
    np.testing.assert_array_equal(host(qs).reshape(s_ref.shape), s_ref)
    kb, kd = key_bytes(keys)
    ref = O.indexer_topk(c_ref.reshape(1, w.n_q, H, d), np.asarray(w_ref).reshape(1, w.n_q, H), kb, kd,
                         host(kscale), 0, w.kv_len, w.k, q_scale=s_ref.reshape(1, w.n_q, H))
    got = host(idx)
    valid_idx_rows(got, 0, w.k)
    ov, worst = overlap(got, ref)
    print(f"overlap {ov:.6f} worst row {worst:.6f}")
    assert ov >= 0.999


@pytest.mark.parametrize("kv_len", [70_001, 200_001])
def test_decode_shape_long_rows(ix, kv_len):
    """Decode-shaped calls (a few sequences, one new row each, long contexts):
    the score kernel widens the codes and runs the top-k's wave-local stage;
    positions bit for bit on integer inputs."""
    w = BASE.with_(name=f"fp8q_decode_{kv_len}", batch=4, n_q=1, q_start=kv_len - 1, kv_len=kv_len, k=2048)
    inputs = _inputs(w)
    got = _run(ix, w, 0, inputs)
    valid_idx_rows(got, w.q_start, w.k)
    np.testing.assert_array_equal(got, _oracle(w, inputs))


@pytest.mark.parametrize("path", [1, 2])
def test_sequences_of_different_lengths(ix, path):
    """Per-sequence starts (ix_problem.seq_q_start) with fp8 queries: row t of
    sequence b sits at starts[b] + t; positions bit for bit."""
    starts = [0, 437, 1200]
    w = BASE.with_(name="fp8q_varlen", batch=3, n_q=190, q_start=max(starts), kv_len=1390, k=300)
    q, qs, wt, keys, scale = _inputs(w)
    idx = torch.full((w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[ix8 varlen] starts={starts} path={path}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, path=path,
                       seq_q_start=torch.tensor(starts, dtype=torch.int64, device="cuda"), q_scale=qs)
    torch.cuda.synchronize()
    kb, kd = key_bytes(keys)
    ref = O.indexer_topk(host(q), host(wt), kb, kd, host(scale), np.array(starts), w.kv_len, w.k,
                         q_scale=host(qs))
    np.testing.assert_array_equal(host(idx), ref)
