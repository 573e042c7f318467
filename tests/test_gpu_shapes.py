"""Every kernel instance the library dispatches to, at small sizes, against
the CPU oracle: indexer key widths d = 16..128 (the fused path takes d in
{16, 32, 64, 128}; the materialised path every multiple of 16), head counts
that leave the second 32-head tile partly empty, and every supported
attention shape with 1, 5 and 16 heads on both work splits (one wave per row
for many rows; four waves and several slot ranges per row for few rows),
with a k that is not a multiple of the 16-slot step."""
import math

import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes, valid_idx_rows
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


def _indexer_case(ix, w, path, rows):
    q, wt = synth.indexer_queries(w, "cuda", 0)
    keys, scale = synth.indexer_keys(w, "cuda", 0)
    idx = torch.full((w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[shapes] indexer H={w.ix_heads} d={w.ix_dim} keys={w.key_dtype} path={path} n_q={w.n_q} "
          f"q_start={w.q_start} k={w.k}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len, path=path)
    torch.cuda.synchronize()
    got = host(idx)
    valid_idx_rows(got, w.q_start, w.k)
    kb, kd = key_bytes(keys)
    want = O.indexer_topk(bits16(q), host(wt), kb, kd, host(scale), w.q_start, w.kv_len, w.k, rows=rows)
    np.testing.assert_array_equal(got[:, rows], want)


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("d,H", [(16, 1), (48, 8), (80, 40), (96, 64), (112, 33), (128, 40)])
def test_materialised_indexer_every_width(ix, d, H, key_dtype):
    w = synth.DECODE_B32.with_(name=f"shape_m{d}_{H}", batch=2, n_q=3, q_start=3000, kv_len=3003, kv_cap=3010,
                               k=256, ix_heads=H, ix_dim=d, key_dtype=key_dtype, mode="exact")
    _indexer_case(ix, w, 2, [0, 1, 2])


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_fused_indexer_partial_head_tile(ix, d, key_dtype):
    w = synth.L16K.with_(name=f"shape_f{d}", n_q=300, q_start=700, kv_len=1000, k=128, ix_heads=40, ix_dim=d,
                         key_dtype=key_dtype, mode="exact")
    _indexer_case(ix, w, 1, [0, 1, 63, 64, 65, 298, 299])


def _attn_case(ix, w, rows):
    g = torch.Generator(device="cuda").manual_seed(w.n_q * 7 + w.q_heads)
    q = synth.attn_queries(w, "cuda", 0)
    kv = synth.latent_kv(w, "cuda", 0)
    n = w.kv_len
    # k slots per row: ascending distinct positions <= the row's own, holes of -1
    idx = torch.full((w.batch, w.n_q, w.k), -1, dtype=torch.int32, device="cuda")
    for t in range(w.n_q):
        p = w.q_start + t
        m = min(w.k - 3, p + 1)
        sel = torch.randperm(p + 1, generator=g, device="cuda")[:m].sort().values.to(torch.int32)
        idx[:, t, :m] = sel
    out = torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.n_q, w.q_heads), device="cuda")
    print(f"[shapes] attention D={w.d_qk} Dv={w.d_v} Hq={w.q_heads} rows={w.batch * w.n_q} k={w.k}", flush=True)
    ix.ix_sparse_attn(q, kv, idx, out, lse=lse, q_start=w.q_start, kv_len=n)
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(w.d_qk)
    o_ref, l_ref = O.sparse_attention(bits16(q), bits16(kv), host(idx), n, sm, w.d_v, rows=rows)
    o = out.float().cpu().numpy()[:, rows]
    err = np.abs(o - o_ref).max()
    assert err <= 2e-2, err
    np.testing.assert_allclose(host(lse)[:, rows], l_ref, rtol=0, atol=1e-3)


SHAPES = [(576, 512), (128, 96), (128, 128), (64, 64)]


@pytest.mark.parametrize("hq", [1, 5, 16])
@pytest.mark.parametrize("dqk,dv", SHAPES)
def test_attention_few_rows(ix, dqk, dv, hq):
    """Four rows: four waves per (row, slot range), two ranges (k = 612)."""
    w = synth.DECODE_B32.with_(name=f"shape_a{dqk}_{hq}", batch=2, n_q=2, q_start=700, kv_len=702, kv_cap=710,
                               k=612, q_heads=hq, d_qk=dqk, d_v=dv)
    _attn_case(ix, w, [0, 1])


@pytest.mark.parametrize("dqk,dv", SHAPES)
def test_attention_many_rows(ix, dqk, dv):
    """1100 rows: one wave per row."""
    w = synth.L16K.with_(name=f"shape_am{dqk}", n_q=1100, q_start=0, kv_len=1100, k=100, q_heads=5, d_qk=dqk,
                         d_v=dv)
    _attn_case(ix, w, [0, 1, 98, 99, 100, 547, 1099])
