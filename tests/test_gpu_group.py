"""GPU checks of the IndexShare layer-group schedule ("IndexShare", LLM
Architecture Gallery, section "How IndexShare Works"): shared layers attend
over the full layer's positions byte for byte, the indexer runs once per full
layer, and all-full with identical indexer inputs reproduces full+shared."""
import math

import numpy as np
import pytest
import torch

from helpers import bits16, ensure_lib, host, key_bytes
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


def _layers(w, roles, same_indexer_per_group=False):
    ixl, atl = [], []
    for l, r in enumerate(roles):
        src = l - (l % 4) if same_indexer_per_group else l
        if r == "F" or same_indexer_per_group:
            q, wt = synth.indexer_queries(w, "cuda", src)
            keys, scale = synth.indexer_keys(w, "cuda", src)
            ixl.append(dict(q=q, w=wt, keys=keys, k_scale=scale))
        else:
            ixl.append(None)
        out = torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.batch, w.n_q, w.q_heads), device="cuda")
        atl.append(dict(q=synth.attn_queries(w, "cuda", l), kv=synth.latent_kv(w, "cuda", l),
                        out=out, lse=lse))
    return ixl, atl


def _group(ix, w, roles, ixl, atl):
    mask = sum(1 << i for i, r in enumerate(roles) if r == "F")
    idx = torch.full((roles.count("F"), w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[group] {w.name} roles={roles} n_q={w.n_q} k={w.k}", flush=True)
    ix.ix_group_forward(ixl, atl, mask, idx, q_start=w.q_start, kv_len=w.kv_len)
    torch.cuda.synchronize()
    return idx


def test_fsss_matches_standalone_calls_and_oracle(ix):
    w = synth.TINY_L1K
    ixl, atl = _layers(w, "FSSS")
    idx = _group(ix, w, "FSSS", ixl, atl)
    before = idx.clone()
    # the F slot equals a standalone indexer call, bit for bit
    solo = torch.empty_like(idx[0])
    e = ixl[0]
    ix.ix_indexer_topk(e["q"], e["w"], e["keys"], solo, k_scale=e["k_scale"], q_start=w.q_start,
                       kv_len=w.kv_len)
    torch.cuda.synchronize()
    assert torch.equal(solo, idx[0])
    # every layer's output equals a standalone attention over that slot, bit for bit
    for l in range(4):
        out = torch.empty_like(atl[l]["out"])
        ix.ix_sparse_attn(atl[l]["q"], atl[l]["kv"], idx[0], out, q_start=w.q_start, kv_len=w.kv_len)
        torch.cuda.synchronize()
        assert torch.equal(out, atl[l]["out"]), f"layer {l}"
    assert torch.equal(before, idx)
    # against the oracle's whole-group walk
    kb, kd = key_bytes(e["keys"])
    ix_in = [(bits16(e["q"]), host(e["w"]), kb, kd, host(e["k_scale"]))] + [None] * 3
    at_in = [(bits16(a["q"]), bits16(a["kv"])) for a in atl]
    rows = list(range(0, w.n_q, 7)) + [w.n_q - 1]
    ref = O.group_forward("FSSS", ix_in, at_in, w.q_start, w.kv_len, w.k, 1.0 / math.sqrt(w.d_qk),
                          w.d_v, rows=rows)
    assert ref["n_indexer_runs"] == 1
    np.testing.assert_array_equal(host(idx[0])[:, rows], ref["idx"][0])
    for l in range(4):
        err = np.abs(atl[l]["out"].float().cpu().numpy()[:, rows] - ref["O"][l]).max()
        assert err <= 2e-2, (l, err)


def test_all_full_with_shared_inputs_equals_fsss(ix):
    w = synth.TINY_L1K.with_(name="allF_eq", mode="float", n_q=777, kv_len=777, k=128)
    roles = "FSSSFSSS"
    ixl, atl = _layers(w, roles, same_indexer_per_group=True)
    idx_fs = _group(ix, w, roles, ixl, atl)
    outs_fs = [a["out"].clone() for a in atl]
    idx_ff = _group(ix, w, "F" * 8, ixl, atl)
    for l in range(8):
        assert torch.equal(idx_ff[l], idx_fs[l // 4]), f"idx layer {l}"
        assert torch.equal(atl[l]["out"], outs_fs[l]), f"out layer {l}"


def test_group_is_deterministic(ix):
    w = synth.L16K.with_(name="determinism", n_q=2100, kv_len=2100, key_dtype="fp8")
    ixl, atl = _layers(w, "FSSS")
    idx1 = _group(ix, w, "FSSS", ixl, atl)
    o1 = [a["out"].clone() for a in atl]
    idx2 = _group(ix, w, "FSSS", ixl, atl)
    assert torch.equal(idx1, idx2)
    for l in range(4):
        assert torch.equal(o1[l], atl[l]["out"])


def test_decode_shape_group(ix):
    """Decode in miniature: several sequences, one new query each, long
    cached context (materialised-score path and split attention)."""
    w = synth.DECODE_B32.with_(name="decode_small", batch=4, q_start=6000, kv_len=6001, kv_cap=6010,
                               mode="exact")
    ixl, atl = _layers(w, "FSSS")
    idx = _group(ix, w, "FSSS", ixl, atl)
    e = ixl[0]
    kb, kd = key_bytes(e["keys"])
    ref_idx = O.indexer_topk(bits16(e["q"]), host(e["w"]), kb, kd, host(e["k_scale"]), w.q_start,
                             w.kv_len, w.k)
    np.testing.assert_array_equal(host(idx[0]), ref_idx)
    for l in range(4):
        ref, _ = O.sparse_attention(bits16(atl[l]["q"]), bits16(atl[l]["kv"]), host(idx[0]), w.kv_len,
                                    1.0 / math.sqrt(w.d_qk), w.d_v)
        assert np.abs(atl[l]["out"].float().cpu().numpy() - ref).max() <= 2e-2


@pytest.mark.parametrize("roles", ["FFSS", "FSFS", "FFFSSS", "FFSSSFSFSSS", "FSSSSSSF"])
def test_irregular_masks_against_oracle(ix, roles):
    """Masks with full layers after shared ones and irregular starts (the
    released pattern repeats F,S,S,S after a few initial exceptions: "GLM-5.2
    and IndexShare for Long-Context Sparse Attention", section "What IndexShare
    reuses"; any F/S assignment is allowed: "IndexShare", section "Why Reusing
    Indices Can Work").  Each F layer's slot is bit-exact against the oracle
    (exact mode), every layer attends over the slot of the most recent F layer
    (the oracle's `used` map), byte for byte as a standalone call over that
    slot, and its output is within 2e-2 of the oracle's."""
    w = synth.TINY_L1K.with_(name=f"mask_{roles}", n_q=300, kv_len=300, k=48)
    ixl, atl = _layers(w, roles)
    idx = _group(ix, w, roles, ixl, atl)
    ix_in, at_in = [], []
    for l, r in enumerate(roles):
        e = ixl[l]
        if r == "F":
            kb, kd = key_bytes(e["keys"])
            ix_in.append((bits16(e["q"]), host(e["w"]), kb, kd, host(e["k_scale"])))
        else:
            ix_in.append(None)
        at_in.append((bits16(atl[l]["q"]), bits16(atl[l]["kv"])))
    rows = list(range(0, w.n_q, 3)) + [w.n_q - 1]
    ref = O.group_forward(roles, ix_in, at_in, w.q_start, w.kv_len, w.k, 1.0 / math.sqrt(w.d_qk), w.d_v,
                          rows=rows)
    assert ref["n_indexer_runs"] == roles.count("F")
    expect_used = [roles[:l + 1].count("F") - 1 for l in range(len(roles))]
    assert ref["used"] == expect_used
    for f in range(roles.count("F")):
        np.testing.assert_array_equal(host(idx[f])[:, rows], ref["idx"][f], err_msg=f"slot {f}")
    for l in range(len(roles)):
        solo = torch.empty_like(atl[l]["out"])
        ix.ix_sparse_attn(atl[l]["q"], atl[l]["kv"], idx[expect_used[l]], solo, q_start=w.q_start,
                          kv_len=w.kv_len)
        torch.cuda.synchronize()
        assert torch.equal(solo, atl[l]["out"]), f"layer {l} did not attend over slot {expect_used[l]}"
        err = np.abs(atl[l]["out"].float().cpu().numpy()[:, rows] - ref["O"][l]).max()
        assert err <= 2e-2, (l, err)


@pytest.mark.parametrize("roles", ["FSSS", "FSFSS", "FFSSF"])
def test_chained_split_merges_equal_standalone_calls(ix, roles):
    """Decode-shaped groups (few rows, so each attention launch splits the
    slots and merges partials): inside the group a layer's partials are merged
    by the next layer's launch, or by a merge kernel before a full layer's
    indexer and after the last layer.  Every layer's output and lse must equal
    a standalone ix_sparse_attn over the same slot, bit for bit; one layer
    passes no lse buffer."""
    w = synth.DECODE_B32.with_(name=f"decode_chain_{roles}", batch=6, q_start=5000, kv_len=5001,
                               kv_cap=5001, roles=roles)
    ixl, atl = _layers(w, roles)
    atl[2]["lse"] = None
    idx = _group(ix, w, roles, ixl, atl)
    f_slot = -1
    for l, r in enumerate(roles):
        f_slot += r == "F"
        out = torch.empty_like(atl[l]["out"])
        lse = None if atl[l]["lse"] is None else torch.empty_like(atl[l]["lse"])
        ix.ix_sparse_attn(atl[l]["q"], atl[l]["kv"], idx[f_slot], out, lse=lse, q_start=w.q_start,
                          kv_len=w.kv_len)
        torch.cuda.synchronize()
        assert torch.equal(out, atl[l]["out"]), f"layer {l}"
        if lse is not None:
            assert torch.equal(lse, atl[l]["lse"]), f"layer {l} lse"


@pytest.mark.parametrize("splits", [2, 3])
def test_forced_splits_on_many_rows_merge_by_kernel(ix, splits):
    """Many rows (one wave per row and split) with the slots forced into
    several splits: such launches cannot merge an earlier layer's partials in
    their prologue, so the group merges each layer's with the merge kernel;
    outputs and lse equal standalone calls with the same split count, bit
    for bit."""
    w = synth.TINY_L1K.with_(name=f"group_splits_{splits}", k=256)
    roles = "FSSFS"
    w = w.with_(roles=roles)
    ixl, atl = _layers(w, roles)
    mask = sum(1 << i for i, r in enumerate(roles) if r == "F")
    idx = torch.full((roles.count("F"), w.batch, w.n_q, w.k), -7, dtype=torch.int32, device="cuda")
    print(f"[group] {w.name} roles={roles} kv_splits={splits}", flush=True)
    ix.ix_group_forward(ixl, atl, mask, idx, q_start=w.q_start, kv_len=w.kv_len, kv_splits=splits)
    torch.cuda.synchronize()
    f_slot = -1
    for l, r in enumerate(roles):
        f_slot += r == "F"
        out = torch.empty_like(atl[l]["out"])
        lse = torch.empty_like(atl[l]["lse"])
        ix.ix_sparse_attn(atl[l]["q"], atl[l]["kv"], idx[f_slot], out, lse=lse, q_start=w.q_start,
                          kv_len=w.kv_len, kv_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, atl[l]["out"]), f"layer {l}"
        assert torch.equal(lse, atl[l]["lse"]), f"layer {l} lse"
