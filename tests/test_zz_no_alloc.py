"""ix_group_forward_noalloc, the layer-group call that allocates nothing (its
kernels work in the library's static device scratch), against
ix_group_forward byte for byte: two calls in a row, the second with a smaller
input, on the decode shape (score rows, row-select state and split-attention
partials in the scratch) and on a small prefill (fused indexer: candidate
buffers and staged keys in the scratch); a call too large for the scratch is
refused before anything runs.  Collected last: its name sorts after every
other test file."""
import pytest
import torch

from helpers import ensure_lib
import ix_synth as synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _inputs(w, tag):
    ixl, atl = [], []
    for l, r in enumerate(w.roles):
        if r == "F":
            q, wt = synth.indexer_queries(w, "cuda", l + tag)
            keys, scale = synth.indexer_keys(w, "cuda", l + tag)
            ixl.append(dict(q=q, w=wt, keys=keys, k_scale=scale))
        else:
            ixl.append(None)
        atl.append(dict(q=synth.attn_queries(w, "cuda", l + tag), kv=synth.latent_kv(w, "cuda", l + tag),
                        out=torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device="cuda"),
                        lse=torch.empty((w.batch, w.n_q, w.q_heads), device="cuda")))
    return ixl, atl


def _both(ix, w, tag):
    """(idx, outs, lses) of ix_group_forward, then of the no-alloc call on
    the same inputs (outputs poisoned in between)."""
    ixl, atl = _inputs(w, tag)
    n_f = w.roles.count("F")
    print(f"[noalloc] {w.name} B={w.batch} n_q={w.n_q} kv_len={w.kv_len} k={w.k} roles={w.roles}", flush=True)
    res = []
    for fn in (ix.ix_group_forward, ix.ix_group_forward_noalloc):
        idx = torch.full((n_f, w.batch, w.n_q, w.k), -9, dtype=torch.int32, device="cuda")
        for a in atl:
            a["out"].fill_(float("nan"))
            a["lse"].fill_(float("nan"))
        fn(ixl, atl, w.f_mask, idx, q_start=w.q_start, kv_len=w.kv_len)
        torch.cuda.synchronize()
        res.append((idx, [a["out"].clone() for a in atl], [a["lse"].clone() for a in atl]))
    return res


def _same(res):
    (i0, o0, l0), (i1, o1, l1) = res
    assert torch.equal(i0, i1)
    for a, b in zip(o0 + l0, o1 + l1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape", ["decode", "prefill"])
def test_noalloc_matches_group_forward_twice_second_smaller(ix, shape):
    if shape == "decode":
        big = synth.DECODE_B32.with_(name="noalloc_big", batch=12, q_start=90000, kv_len=90001, kv_cap=90016)
        small = synth.DECODE_B32.with_(name="noalloc_small", batch=5, q_start=31000, kv_len=31001,
                                       kv_cap=31008, mode="exact")
    else:
        big = synth.TINY_L1K.with_(name="noalloc_big", n_q=1024, kv_len=1024, roles="FSSSFSSS")
        small = synth.L16K.with_(name="noalloc_small", n_q=700, kv_len=900, q_start=200, k=512,
                                 key_dtype="fp8", mode="exact")
    for w, tag in ((big, 0), (small, 20)):
        _same(_both(ix, w, tag))


def test_noalloc_refuses_a_call_beyond_the_scratch(ix):
    """The fused path at 4096 rows with k = 2048 needs 128 MiB of candidate
    buffers: refused with IX_E_WORKSPACE, nothing written."""
    w = synth.L16K.with_(name="noalloc_too_big", n_q=4096, kv_len=4096)
    ixl, atl = _inputs(w, 40)
    idx = torch.full((1, 1, w.n_q, w.k), -9, dtype=torch.int32, device="cuda")
    with pytest.raises(ix.IxError) as e:
        ix.ix_group_forward_noalloc(ixl, atl, w.f_mask, idx, q_start=0, kv_len=w.kv_len)
    assert e.value.status == ix.IX_E_WORKSPACE and "needs" in str(e.value)
    torch.cuda.synchronize()
    assert bool((idx == -9).all())
