"""MTP draft steps with index reuse ("GLM-5.2 and IndexShare for Long-Context
Sparse Attention", section "Reuse in the MTP layer") on the GPU against the
oracle.  The first draft step runs ix_indexer_topk and attends; every later
step calls ix_sparse_attn with the same index buffer, the same problem and the
same KV cache.  The cache already holds rows past the first step's position,
so a step that selected again, or read rows it was not given, would differ."""
import math

import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes
import ix_synth as synth
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

STEPS = 4


@pytest.fixture(scope="module")
def ix():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_lib()
    import long_context_sparse_ix_amd as m
    return m


def _inputs(w):
    q, wt = synth.indexer_queries(w, "cuda", 0)
    keys, scale = synth.indexer_keys(w, "cuda", 0)
    kv = synth.latent_kv(w, "cuda", 0)
    drafts = [synth.attn_queries(w, "cuda", 0, step=j) for j in range(STEPS)]
    return (q, wt, keys, scale), kv, drafts


def _draft_calls(ix, w, ixin, kv, drafts, seq_q_start=None):
    q, wt, keys, scale = ixin
    idx = torch.full((w.batch, 1, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[mtp] {w.name} B={w.batch} pos={w.q_start} kv_len={w.kv_len} steps={STEPS}", flush=True)
    ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len,
                       seq_q_start=seq_q_start)
    before = idx.clone()
    outs = []
    for Q in drafts:
        out = torch.empty((w.batch, 1, w.q_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
        ix.ix_sparse_attn(Q, kv, idx, out, q_start=w.q_start, kv_len=w.kv_len)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(before, idx)          # the later steps leave the positions untouched
    return idx, outs


def _oracle(w, ixin, kv, drafts, starts):
    q, wt, keys, scale = ixin
    kb, kd = key_bytes(keys)
    return O.mtp_draft((bits16(q), host(wt), kb, kd, host(scale)), [bits16(d) for d in drafts], bits16(kv),
                       starts, w.kv_len, w.k, 1.0 / math.sqrt(w.d_qk), w.d_v)


def test_draft_steps_reuse_the_first_steps_positions(ix):
    w = synth.DECODE_B32.with_(name="mtp_draft", batch=4, q_start=5000, kv_len=5000 + STEPS, kv_cap=5064,
                               mode="exact")
    ixin, kv, drafts = _inputs(w)
    idx, outs = _draft_calls(ix, w, ixin, kv, drafts)
    ref = _oracle(w, ixin, kv, drafts, w.q_start)
    assert ref["n_indexer_runs"] == 1
    np.testing.assert_array_equal(host(idx), ref["idx"])
    assert host(idx).max() <= w.q_start        # nothing past the first step's position
    for j in range(STEPS):
        err = np.abs(outs[j].float().cpu().numpy() - ref["O"][j]).max()
        assert err <= 2e-2, (j, err)
    assert not torch.equal(outs[0], outs[1])   # each step has its own queries


def test_draft_steps_equal_a_group_with_one_full_layer_over_one_cache(ix):
    """The same draft steps through ix_group_forward: layer 0 full, the rest
    shared, every layer's attention over the one cache -- byte for byte the
    step-by-step calls."""
    w = synth.DECODE_B32.with_(name="mtp_group", batch=3, q_start=3000, kv_len=3000 + STEPS, kv_cap=3010,
                               mode="exact")
    ixin, kv, drafts = _inputs(w)
    idx, outs = _draft_calls(ix, w, ixin, kv, drafts)
    q, wt, keys, scale = ixin
    ixl = [dict(q=q, w=wt, keys=keys, k_scale=scale)] + [None] * (STEPS - 1)
    atl = [dict(q=d, kv=kv, out=torch.empty_like(outs[0])) for d in drafts]
    gidx = torch.full((1, w.batch, 1, w.k), -7, dtype=torch.int32, device="cuda")
    ix.ix_group_forward(ixl, atl, 1, gidx, q_start=w.q_start, kv_len=w.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(gidx[0], idx)
    for j in range(STEPS):
        assert torch.equal(atl[j]["out"], outs[j]), j


def test_draft_steps_for_sequences_of_different_lengths(ix):
    starts = [6000, 100, 2047, 4321]
    w = synth.DECODE_B32.with_(name="mtp_varlen", batch=4, q_start=6000, kv_len=6000 + STEPS, kv_cap=6010,
                               mode="exact")
    ixin, kv, drafts = _inputs(w)
    seq = torch.tensor(starts, dtype=torch.int64, device="cuda")
    idx, outs = _draft_calls(ix, w, ixin, kv, drafts, seq_q_start=seq)
    ref = _oracle(w, ixin, kv, drafts, starts)
    np.testing.assert_array_equal(host(idx), ref["idx"])
    for j in range(STEPS):
        err = np.abs(outs[j].float().cpu().numpy() - ref["O"][j]).max()
        assert err <= 2e-2, (j, err)
