"""The C-ABI library on the CPU: it loads, exports every symbol ix.h declares,
its struct layout matches the Python binding, and argument validation rejects
bad calls before any HIP work (no compute is launched here)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from helpers import ROOT, ensure_lib
import long_context_sparse_ix_amd as ix

HEADER = os.path.join(ROOT, "include", "ix.h")
DUMMY = 0x10000          # aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(ix_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    ensure_lib()
    names = declared_functions()
    assert {"ix_indexer_topk", "ix_sparse_attn", "ix_group_forward", "ix_topk_scores",
            "ix_workspace_bytes", "ix_status_str", "ix_abi_version", "ix_last_error",
            "ix_index_overlap", "ix_append_keys", "ix_indexer_argmax",
            "ix_group_forward_noalloc", "ix_indexer_project", "ix_quantize_queries"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", ix.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(ix_\w+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported
    lib = ctypes.CDLL(ix.LIB_PATH)
    for n in names:
        getattr(lib, n)


def test_struct_layout_matches_header():
    """Compile a probe against ix.h with gcc and compare sizes/offsets with
    the ctypes mirrors."""
    probe = r"""
#include <stdio.h>
#include <stddef.h>
#include "ix.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("ix_problem %zu\nix_indexer_in %zu\nix_attn_in %zu\nix_group_desc %zu\nix_project_in %zu\n",
         sizeof(ix_problem), sizeof(ix_indexer_in), sizeof(ix_attn_in), sizeof(ix_group_desc),
         sizeof(ix_project_in));
  F(ix_problem, q_start) F(ix_problem, kv_cap) F(ix_problem, k) F(ix_problem, seq_q_start)
  F(ix_indexer_in, q) F(ix_indexer_in, k_scale) F(ix_indexer_in, path)
  F(ix_indexer_in, q_dtype) F(ix_indexer_in, reserved) F(ix_indexer_in, q_scale)
  F(ix_attn_in, sm_scale) F(ix_attn_in, kv_splits) F(ix_attn_in, q) F(ix_attn_in, lse)
  F(ix_group_desc, f_mask) F(ix_group_desc, ixr) F(ix_group_desc, attn)
  F(ix_project_in, d_in) F(ix_project_in, reserved) F(ix_project_in, x) F(ix_project_in, w_proj)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write(probe)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        lines = dict(l.split() for l in subprocess.run([exe], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    m = {"ix_problem": ix.Problem, "ix_indexer_in": ix.IndexerIn, "ix_attn_in": ix.AttnIn,
         "ix_group_desc": ix.GroupDesc, "ix_project_in": ix.ProjectIn}
    for k, v in lines.items():
        if "." in k:
            s, f = k.split(".")
            assert getattr(m[s], f).offset == int(v), k
        else:
            assert ctypes.sizeof(m[k]) == int(v), k


def _prob(**kw):
    base = dict(batch=1, n_q=8, q_start=0, kv_len=8, kv_cap=8, k=4, reserved=0)
    base.update(kw)
    return ix.Problem(**base)


def _ixr(**kw):
    base = dict(heads=4, dim=32, k_dtype=ix.IX_DTYPE_BF16, path=0, q=DUMMY, w=DUMMY, k=DUMMY, k_scale=None,
                q_dtype=0, reserved=0, q_scale=None)
    base.update(kw)
    return ix.IndexerIn(**base)


def _att(**kw):
    base = dict(q_heads=8, d_qk=128, d_v=96, sm_scale=0.0, kv_splits=0, reserved=0, q=DUMMY,
                kv=DUMMY, out=DUMMY, lse=None)
    base.update(kw)
    return ix.AttnIn(**base)


def _call_ix(p, d, idx=DUMMY, ws=None, nb=0):
    lib = ensure_lib()
    return lib.ix_indexer_topk(ctypes.byref(p), ctypes.byref(d), idx, ws, nb, None)


def _call_att(p, d, idx=DUMMY, ws=None, nb=0):
    lib = ensure_lib()
    return lib.ix_sparse_attn(ctypes.byref(p), ctypes.byref(d), idx, ws, nb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), ix.IX_E_SHAPE), (dict(k=4096), ix.IX_E_SHAPE), (dict(batch=0), ix.IX_E_SHAPE),
    (dict(kv_len=7), ix.IX_E_SHAPE), (dict(kv_cap=7), ix.IX_E_SHAPE),
    (dict(q_start=-1), ix.IX_E_SHAPE), (dict(reserved=1), ix.IX_E_SHAPE),
    (dict(seq_q_start=DUMMY + 4), ix.IX_E_SHAPE),  # per-sequence starts: int64, 8-byte aligned
])
def test_problem_validation(kw, status):
    assert _call_ix(_prob(**kw), _ixr()) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ix.IX_E_NULL), (dict(k=None), ix.IX_E_NULL), (dict(w=None), ix.IX_E_NULL),
    (dict(k_dtype=7), ix.IX_E_DTYPE), (dict(k_dtype=ix.IX_DTYPE_FP8_E4M3FN), ix.IX_E_NULL),
    (dict(k_scale=DUMMY), ix.IX_E_SHAPE), (dict(heads=65), ix.IX_E_SHAPE),
    (dict(dim=24), ix.IX_E_SHAPE), (dict(dim=144), ix.IX_E_SHAPE), (dict(path=3), ix.IX_E_SHAPE),
    (dict(q=DUMMY + 8), ix.IX_E_SHAPE), (dict(dim=48, path=1), ix.IX_E_SHAPE),
    # fp8 queries: a known query dtype, their scale present exactly when they are fp8
    (dict(q_dtype=3), ix.IX_E_DTYPE), (dict(q_dtype=ix.IX_DTYPE_FP8_E4M3FN), ix.IX_E_NULL),
    (dict(q_scale=DUMMY), ix.IX_E_SHAPE), (dict(q_dtype=ix.IX_DTYPE_BF16, q_scale=DUMMY), ix.IX_E_SHAPE),
    (dict(q_dtype=ix.IX_DTYPE_FP8_E4M3FN, q_scale=DUMMY + 4), ix.IX_E_SHAPE),
    (dict(reserved=1), ix.IX_E_SHAPE),
])
def test_indexer_validation(kw, status):
    assert _call_ix(_prob(), _ixr(**kw)) == status


def test_fp8_query_workspace():
    """fp8 queries with fp8 keys and d in {64, 128} read the key cache in
    place: the fused path's workspace is the candidate buffers alone, while
    the other forms also hold a staged bf16 copy of the keys."""
    p = _prob(n_q=256, kv_len=4096, kv_cap=4096, k=512)
    f8 = ix.IX_DTYPE_FP8_E4M3FN
    cand = 256 * 1024 * 8          # per row: k + max(k, 256) candidate slots of 8 bytes
    for dim in (64, 128):
        fast = ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_TOPK,
                                     _ixr(dim=dim, k_dtype=f8, k_scale=DUMMY, q_dtype=f8, q_scale=DUMMY))
        staged = ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_TOPK, _ixr(dim=dim, k_dtype=f8, k_scale=DUMMY))
        assert staged - fast >= 4096 * dim * 2                   # the staged key copy
        assert fast == cand
        # the top-1 entry point needs no workspace at all in that form
        assert ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_ARGMAX,
                                     _ixr(dim=dim, k_dtype=f8, k_scale=DUMMY, q_dtype=f8, q_scale=DUMMY)) == 0
    # bf16 keys with fp8 queries: widened form, keys staged as before
    wide = ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_TOPK, _ixr(dim=128, q_dtype=f8, q_scale=DUMMY))
    assert wide == ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_TOPK, _ixr(dim=128))


def test_indexer_null_idx_and_workspace():
    assert _call_ix(_prob(), _ixr(), idx=None) == ix.IX_E_NULL
    # few rows -> materialised path needs a score workspace
    assert _call_ix(_prob(), _ixr(), ws=None, nb=0) == ix.IX_E_WORKSPACE
    need = ix.ix_workspace_bytes(_prob(), ix.IX_OP_INDEXER_TOPK, _ixr())
    assert need >= 8 * 8 * 4
    assert _call_ix(_prob(), _ixr(), ws=None, nb=need) == ix.IX_E_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(q_heads=17), ix.IX_E_SHAPE), (dict(d_qk=256), ix.IX_E_SHAPE),
    (dict(d_v=100), ix.IX_E_SHAPE), (dict(kv_splits=65), ix.IX_E_SHAPE),
    (dict(out=None), ix.IX_E_NULL), (dict(kv=None), ix.IX_E_NULL), (dict(reserved=2), ix.IX_E_SHAPE),
    (dict(sm_scale=float("nan")), ix.IX_E_SHAPE),
])
def test_attention_validation(kw, status):
    assert _call_att(_prob(), _att(**kw)) == status


def test_attention_split_workspace_is_checked():
    p = _prob(n_q=2, kv_len=4096, kv_cap=4096, q_start=0, k=2048)
    need = ix.ix_workspace_bytes(p, ix.IX_OP_SPARSE_ATTN, _att(kv_splits=8))
    assert need >= 2 * 8 * 16 * 96 * 4
    assert _call_att(p, _att(kv_splits=8)) == ix.IX_E_WORKSPACE


def test_group_role_mask_validation():
    lib = ensure_lib()
    p = _prob()
    ixr = (ix.IndexerIn * 4)(*[_ixr() for _ in range(4)])
    att = (ix.AttnIn * 4)(*[_att() for _ in range(4)])
    call = lambda n, mask: lib.ix_group_forward(ctypes.byref(p), n, mask, ixr, att, DUMMY, None, 0, None)
    assert call(4, 0b1110) == ix.IX_E_ROLES          # first layer must be full
    assert call(0, 0b1) == ix.IX_E_ROLES
    assert call(65, 0b1) == ix.IX_E_ROLES
    assert call(4, 0b10001) == ix.IX_E_ROLES          # role bit beyond the last layer
    bad = (ix.AttnIn * 4)(*[_att() for _ in range(3)] + [_att(d_v=100)])
    assert lib.ix_group_forward(ctypes.byref(p), 4, 1, ixr, bad, DUMMY, None, 0, None) == ix.IX_E_SHAPE
    # shared layers' indexer entries are not read: a zeroed entry is fine for
    # validation, which then stops at the missing workspace
    ixr2 = (ix.IndexerIn * 4)(_ixr(), ix.IndexerIn(), ix.IndexerIn(), ix.IndexerIn())
    assert lib.ix_group_forward(ctypes.byref(p), 4, 1, ixr2, att, DUMMY, None, 0, None) == ix.IX_E_WORKSPACE


def test_indexer_argmax_validation():
    """The top-1 entry point: fused path only, outputs 4-byte aligned, the
    staged-key workspace checked before anything is enqueued."""
    lib = ensure_lib()
    p = _prob(n_q=256, kv_len=256, kv_cap=256)
    call = lambda d, pos=DUMMY, score=None, ws=None, nb=0: lib.ix_indexer_argmax(
        ctypes.byref(p), ctypes.byref(d), pos, score, ws, nb, None)
    assert call(_ixr(), pos=None) == ix.IX_E_NULL
    assert call(_ixr(q=None)) == ix.IX_E_NULL
    assert call(_ixr(dim=48)) == ix.IX_E_SHAPE           # no fused kernel for d = 48
    assert call(_ixr(path=ix.IX_PATH_MATERIALIZED)) == ix.IX_E_SHAPE
    assert call(_ixr(), pos=DUMMY + 2) == ix.IX_E_SHAPE
    assert call(_ixr(), score=DUMMY + 1) == ix.IX_E_SHAPE
    assert call(_ixr()) == ix.IX_E_WORKSPACE
    need = ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_ARGMAX, _ixr())
    assert need >= (256 + 64) * 32 * 2                  # the bf16 key copy, one tile of padding
    assert call(_ixr(), ws=None, nb=need) == ix.IX_E_NULL
    assert ix.ix_workspace_bytes(p, ix.IX_OP_INDEXER_ARGMAX, _ixr(dim=48)) == 0


def test_topk_scores_validation():
    lib = ensure_lib()
    p = _prob()
    assert lib.ix_topk_scores(ctypes.byref(p), None, 8, DUMMY, None, 0, None) == ix.IX_E_NULL
    assert lib.ix_topk_scores(ctypes.byref(p), DUMMY, 7, DUMMY, None, 0, None) == ix.IX_E_SHAPE


def test_status_strings():
    for s in range(7):
        assert ix.ix_status_str(s).startswith("IX_")
    assert ix.ix_abi_version() == 7


def test_index_overlap_validation():
    lib = ensure_lib()
    p = _prob()
    assert lib.ix_index_overlap(ctypes.byref(p), None, DUMMY, DUMMY, None) == ix.IX_E_NULL
    assert lib.ix_index_overlap(ctypes.byref(p), DUMMY, DUMMY, None, None) == ix.IX_E_NULL
    assert lib.ix_index_overlap(ctypes.byref(p), DUMMY + 4, DUMMY, DUMMY, None) == ix.IX_E_SHAPE
    bad = _prob(k=0)
    assert lib.ix_index_overlap(ctypes.byref(bad), DUMMY, DUMMY, DUMMY, None) == ix.IX_E_SHAPE


def test_append_keys_validation():
    lib = ensure_lib()
    p = _prob()                                    # kv_cap 8
    call = lambda dim=32, n=1, pos=0, kn=DUMMY, kc=DUMMY, ks=DUMMY: lib.ix_append_keys(
        ctypes.byref(p), dim, kn, n, pos, kc, ks, None)
    assert call(kn=None) == ix.IX_E_NULL
    assert call(ks=None) == ix.IX_E_NULL
    assert call(dim=24) == ix.IX_E_SHAPE
    assert call(dim=144) == ix.IX_E_SHAPE
    assert call(n=-1) == ix.IX_E_SHAPE
    assert call(pos=-1) == ix.IX_E_SHAPE
    assert call(n=3, pos=6) == ix.IX_E_SHAPE         # past kv_cap
    assert call(kn=DUMMY + 8) == ix.IX_E_SHAPE
    assert call(ks=DUMMY + 2) == ix.IX_E_SHAPE



def test_project_validation():
    lib = ensure_lib()

    def call(rows=4, q=DUMMY, w=DUMMY, **kw):
        base = dict(heads=2, dim=16, d_in=64, reserved=0, x=DUMMY, w_proj=DUMMY)
        base.update(kw)
        pin = ix.ProjectIn(**base)
        return lib.ix_indexer_project(rows, ctypes.byref(pin), q, w, None)
    assert lib.ix_indexer_project(4, None, DUMMY, DUMMY, None) == ix.IX_E_NULL
    assert call(x=None) == ix.IX_E_NULL
    assert call(w_proj=None) == ix.IX_E_NULL
    assert call(q=None) == ix.IX_E_NULL
    assert call(w=None) == ix.IX_E_NULL
    assert call(rows=-1) == ix.IX_E_SHAPE
    assert call(heads=0) == ix.IX_E_SHAPE
    assert call(dim=0) == ix.IX_E_SHAPE
    assert call(d_in=96) == ix.IX_E_SHAPE           # not a multiple of 64
    assert call(d_in=0) == ix.IX_E_SHAPE
    assert call(reserved=1) == ix.IX_E_SHAPE
    assert call(heads=1 << 16, dim=1 << 15) == ix.IX_E_SHAPE
    assert call(d_in=1 << 22) == ix.IX_E_SHAPE       # a 256-row tile would span 2^31 bytes
    assert call(rows=1 << 40) == ix.IX_E_SHAPE       # more tiles than an int counts
    assert call(x=DUMMY + 8) == ix.IX_E_SHAPE
    assert call(w_proj=DUMMY + 8) == ix.IX_E_SHAPE
    assert call(q=DUMMY + 1) == ix.IX_E_SHAPE
    assert call(w=DUMMY + 2) == ix.IX_E_SHAPE
    assert call(rows=0) == ix.IX_OK                 # nothing to do, nothing launched


def test_append_keys_per_sequence_rows_need_pos_at_the_bound():
    """With per-sequence starts each sequence's rows move down by its distance
    below q_start, so pos < q_start (a negative row) is rejected."""
    lib = ensure_lib()
    p = _prob(n_q=1, q_start=5, kv_len=8, seq_q_start=DUMMY)
    call = lambda pos, n=1: lib.ix_append_keys(ctypes.byref(p), 32, DUMMY, n, pos, DUMMY, DUMMY, None)
    assert call(4) == ix.IX_E_SHAPE
    assert call(8) == ix.IX_E_SHAPE                  # past kv_cap


def test_workspace_sizes_cover_the_row_select_state():
    """Host-side sizes: the few-long-rows top-k needs at least its 8192-entry
    candidate list per row plus one 16-byte record per 1024-score piece; the
    materialised indexer adds the score rows and one 16-byte record per
    640-key wave of the score kernel; many-row calls and rows no longer than
    k need no row-select state."""
    lib = ensure_lib()
    rows, n = 32, 200_001
    p = _prob(batch=rows, n_q=1, q_start=n - 1, kv_len=n, kv_cap=n, k=2048)
    topk = lib.ix_workspace_bytes(ctypes.byref(p), ix.IX_OP_TOPK_SCORES, None)
    pieces = -(-n // 1024)
    assert topk >= rows * 8192 * 8 + rows * pieces * 16
    d = _ixr(heads=64, dim=128, k_dtype=ix.IX_DTYPE_FP8_E4M3FN, path=2, k_scale=DUMMY)
    mat = lib.ix_workspace_bytes(ctypes.byref(p), ix.IX_OP_INDEXER_TOPK, ctypes.byref(d))
    ld = (n + 3) // 4 * 4
    assert mat >= rows * ld * 4 + rows * (-(-n // 640)) * 16 + topk
    many = _prob(batch=1, n_q=1024, q_start=n - 1024, kv_len=n, kv_cap=n, k=2048)
    assert lib.ix_workspace_bytes(ctypes.byref(many), ix.IX_OP_TOPK_SCORES, None) == 0
    short = _prob(batch=4, n_q=1, q_start=1000, kv_len=1001, kv_cap=1001, k=2048)
    assert lib.ix_workspace_bytes(ctypes.byref(short), ix.IX_OP_TOPK_SCORES, None) == 0


def test_group_noalloc_validates_and_rejects_oversized_calls_before_any_hip_call():
    """ix_group_forward_noalloc: argument errors as ix_group_forward, and a
    call whose workspace exceeds the 64 MiB static scratch (the fused path at
    L = 128K needs GiBs) is rejected with IX_E_WORKSPACE and its sizes in
    ix_last_error(), all before any HIP call (this runs without a GPU)."""
    lib = ensure_lib()
    p = _prob(n_q=131072, kv_len=131072, kv_cap=131072, k=2048)
    ixr = (ix.IndexerIn * 4)(*[_ixr(heads=64, dim=128) for _ in range(4)])
    att = (ix.AttnIn * 4)(*[_att() for _ in range(4)])
    call = lambda n, mask, idx=DUMMY, prob=p: lib.ix_group_forward_noalloc(ctypes.byref(prob), n, mask, ixr, att,
                                                                         idx, None)
    gd = ix.GroupDesc(4, 0, 1, ixr, att)
    assert ix.ix_workspace_bytes(p, ix.IX_OP_GROUP_FORWARD, gd) > ix.NOALLOC_SCRATCH_BYTES
    assert call(4, 0b0001) == ix.IX_E_WORKSPACE
    msg = lib.ix_last_error().decode()
    assert "needs" in msg and str(ix.NOALLOC_SCRATCH_BYTES) in msg
    assert call(4, 0b1110) == ix.IX_E_ROLES
    assert call(0, 0b1) == ix.IX_E_ROLES
    assert call(4, 0b1, idx=None) == ix.IX_E_NULL
    assert call(4, 0b1, idx=DUMMY + 4) == ix.IX_E_SHAPE
    assert call(4, 0b1, prob=_prob(k=0)) == ix.IX_E_SHAPE
    bad = (ix.AttnIn * 4)(*[_att() for _ in range(3)] + [_att(d_v=100)])
    assert lib.ix_group_forward_noalloc(ctypes.byref(p), 4, 1, ixr, bad, DUMMY, None) == ix.IX_E_SHAPE


def test_quantize_queries_validation():
    lib = ensure_lib()
    call = lambda n=4, dim=64, q=DUMMY, c=DUMMY, s=DUMMY: lib.ix_quantize_queries(n, dim, q, c, s, None)
    assert call(q=None) == ix.IX_E_NULL
    assert call(c=None) == ix.IX_E_NULL
    assert call(s=None) == ix.IX_E_NULL
    assert call(n=-1) == ix.IX_E_SHAPE
    assert call(dim=8) == ix.IX_E_SHAPE
    assert call(dim=40) == ix.IX_E_SHAPE            # not a multiple of 16
    assert call(dim=144) == ix.IX_E_SHAPE
    assert call(n=1 << 60) == ix.IX_E_SHAPE
    assert call(q=DUMMY + 8) == ix.IX_E_SHAPE
    assert call(c=DUMMY + 8) == ix.IX_E_SHAPE
    assert call(s=DUMMY + 2) == ix.IX_E_SHAPE
