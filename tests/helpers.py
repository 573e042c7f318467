"""Test helpers: byte-exact host copies of device inputs and comparisons."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> host uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bytes8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def host(t):
    return None if t is None else t.detach().cpu().numpy()


def key_bytes(keys: torch.Tensor) -> tuple[np.ndarray, str]:
    if keys.dtype == torch.bfloat16:
        return bits16(keys), "bf16"
    return bytes8(keys), "fp8"


def ensure_lib():
    """Build libix.so if it is missing (tests load what is built)."""
    import long_context_sparse_ix_amd as ix
    if not os.path.exists(ix.LIB_PATH):
        from long_context_sparse_ix_amd import build
        build.build()
    return ix.load()


def overlap(gpu_idx: np.ndarray, ref_idx: np.ndarray):
    """Set overlap of valid positions, summed over rows, and the worst row."""
    g = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    r = ref_idx.reshape(-1, ref_idx.shape[-1])
    inter = tot = 0
    worst = 1.0
    for a, b in zip(g, r):
        sa = set(a[a >= 0].tolist())
        sb = set(b[b >= 0].tolist())
        i = len(sa & sb)
        inter += i
        tot += len(sb)
        if sb:
            worst = min(worst, i / len(sb))
    return inter / max(tot, 1), worst


def valid_idx_rows(idx: np.ndarray, q_start: int, k: int):
    """Structural invariants of an index buffer: ascending valid positions,
    each <= its row's position, then -1 padding; count == min(k, p+1)."""
    rows = idx.reshape(-1, idx.shape[-1])
    n_q = idx.shape[-2]
    for i, row in enumerate(rows):
        p = q_start + (i % n_q)
        n = min(k, p + 1)
        assert np.all(row[n:] == -1), f"row {i}: padding"
        v = row[:n]
        assert np.all(v >= 0) and np.all(v <= p), f"row {i}: out of causal range"
        assert np.all(np.diff(v) > 0), f"row {i}: not strictly ascending"
