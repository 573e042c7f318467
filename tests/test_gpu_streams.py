"""Calls on different streams: the binding keeps one workspace per (device,
stream), allocated on that stream, so two layer groups queued on two streams
at once must give exactly what each gives alone on the default stream."""
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


def _group_inputs(w, tag):
    ixl, atl = [], []
    for l, r in enumerate(w.roles):
        if r == "F":
            q, wt = synth.indexer_queries(w, "cuda", l + tag)
            keys, scale = synth.indexer_keys(w, "cuda", l + tag)
            ixl.append(dict(q=q, w=wt, keys=keys, k_scale=scale))
        else:
            ixl.append(None)
        atl.append(dict(q=synth.attn_queries(w, "cuda", l + tag), kv=synth.latent_kv(w, "cuda", l + tag),
                        out=torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16,
                                        device="cuda")))
    idx = torch.empty((w.roles.count("F"), w.batch, w.n_q, w.k), dtype=torch.int32, device="cuda")
    return ixl, atl, idx


@pytest.mark.parametrize("shape", ["prefill", "decode"])
def test_two_streams_match_one(ix, shape):
    """Prefill-shaped groups (fused indexer: candidate buffers and staged keys
    in the workspace) and decode-shaped ones (score rows, row-select state and
    split-attention partials in the workspace), two of different sizes per
    stream so the larger request replaces a cached buffer."""
    if shape == "prefill":
        wa = synth.L16K.with_(name="streams_a", n_q=1500, kv_len=1500, key_dtype="fp8")
        wb = synth.L16K.with_(name="streams_b", n_q=2600, kv_len=2600)
    else:
        wa = synth.DECODE_B32.with_(name="streams_a", batch=4, q_start=30000, kv_len=30001, kv_cap=30016)
        wb = synth.DECODE_B32.with_(name="streams_b", batch=6, q_start=50000, kv_len=50001, kv_cap=50016)
    runs = [(wa, *_group_inputs(wa, 0)), (wb, *_group_inputs(wb, 10))]
    print(f"[streams] {shape}: single-stream reference", flush=True)
    ref = []
    for w, ixl, atl, idx in runs:
        ix.ix_group_forward(ixl, atl, w.f_mask, idx, q_start=w.q_start, kv_len=w.kv_len)
        torch.cuda.synchronize()
        ref.append((idx.clone(), [a["out"].clone() for a in atl]))
        idx.fill_(-9)
        for a in atl:
            a["out"].zero_()
    torch.cuda.synchronize()
    # the first stream also runs the second workload's group into outputs of
    # its own, so that stream's cached workspace is replaced by a larger one
    wb_, ixl_b, atl_b, _ = runs[1]
    extra_atl = [dict(a, out=torch.empty_like(a["out"])) for a in atl_b]
    extra = (wb_, ixl_b, extra_atl, torch.empty_like(runs[1][3]))
    print(f"[streams] {shape}: two streams, three rounds", flush=True)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for (w, ixl, atl, idx), s in ((runs[0], streams[0]), (runs[1], streams[1]), (extra, streams[0])):
            with torch.cuda.stream(s):
                ix.ix_group_forward(ixl, atl, w.f_mask, idx, q_start=w.q_start, kv_len=w.kv_len, stream=s)
        torch.cuda.synchronize()
        for (w, ixl, atl, idx), (ridx, routs) in zip(runs + [extra], ref + [ref[1]]):
            assert torch.equal(idx, ridx)
            for a, r in zip(atl, routs):
                assert torch.equal(a["out"], r)
        for (w, ixl, atl, idx) in runs + [extra]:
            idx.fill_(-9)
            for a in atl:
                a["out"].zero_()
        torch.cuda.synchronize()
