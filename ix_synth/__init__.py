"""Seeded synthetic inputs for the DSA layer group (indexer + sparse attention).

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds workload shapes and random-number recipes only: none of
the method's arithmetic (no scoring, no selection, no attention) lives here.

Recipe (all draws come from torch generators seeded by ``_seed(...)`` below):

* exact mode (integer-valued, so every fp32 partial sum of the indexer is exact):
  indexer queries and keys are integers drawn uniformly from -8..8 inclusive,
  head weights are drawn uniformly from {1, 2, 4}; an fp8 key is the integer's
  e4m3fn code with a per-row scale of exactly 1.
* float mode: indexer queries ~ N(0, 1/sqrt(d)) rounded to bf16, head weights
  ~ N(0, 1) in fp32; bf16 keys ~ N(0, 1/sqrt(d)); fp8 keys start as N(0, 1)
  fp32 rows, each row is scaled by max|k|/448 and rounded to e4m3fn (RNE,
  saturated to +-448), and that scale is stored next to the codes.
* fp8 indexer queries (a mode the caller declares): exact mode draws
  integers from -8..8 as e4m3fn codes with a per-(row, head) scale 2^e, e
  uniform in {-1, 0, 1}; float mode draws N(0, 1/sqrt(d)) fp32 rows and
  quantises each (row, head) row like an fp8 key row (scale max|q|/448).
  Head weights follow the bf16 recipe.
* attention queries and latent KV rows ~ N(0, 1) rounded to bf16.
* indexer projection (q_I and head weights from hidden states): hidden rows
  ~ N(0, 1) and the stacked weight [H*d + H][d_in] ~ N(0, 1/d_in), both
  rounded to bf16 (exact mode: integers in -8..8); d_in = 6144, the hidden
  width of the GLM-5.2 configuration.

Tensors are generated on the device the caller names (``cpu`` or ``cuda``);
the two devices draw different streams for the same seed, so a test always
generates once and copies the bytes to wherever they are needed.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one DSA layer-group run (every layer shares these sizes)."""

    name: str
    batch: int
    n_q: int                 # query rows per sequence
    q_start: int             # absolute position of query row 0
    kv_len: int              # valid key rows per sequence
    k: int                   # positions kept per query row
    roles: str               # one letter per layer: F (full) or S (shared)
    ix_heads: int
    ix_dim: int
    key_dtype: str           # "bf16" or "fp8"
    q_heads: int
    d_qk: int
    d_v: int
    mode: str = "float"      # "float" or "exact"
    kv_cap: int = 0          # rows allocated per sequence (0 -> kv_len)
    decode_steps: int = 0    # >0: decode workload, one query row per step
    seed: int = 0

    @property
    def cap(self) -> int:
        return self.kv_cap if self.kv_cap else self.kv_len

    @property
    def n_layers(self) -> int:
        return len(self.roles)

    @property
    def f_mask(self) -> int:
        m = 0
        for i, r in enumerate(self.roles):
            if r == "F":
                m |= 1 << i
        return m

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on (the benchmark configurations;
# k=2048 and the 1M context follow the pages).
TINY_L1K = Workload("tiny_l1k_exact", 1, 1024, 0, 1024, 64, "FSSS", 4, 32, "bf16",
                    8, 128, 96, mode="exact")
L16K = Workload("prefill_l16k", 1, 16384, 0, 16384, 2048, "FSSS", 64, 128, "bf16",
                16, 576, 512)
L128K = Workload("prefill_l128k_2groups", 1, 131072, 0, 131072, 2048, "FSSSFSSS", 64, 128,
                 "fp8", 16, 576, 512)
DECODE_B32 = Workload("decode_b32_ctx200k", 32, 1, 200000, 200001, 2048, "FSSS", 64, 128,
                      "fp8", 16, 576, 512, kv_cap=200064, decode_steps=64)
CHUNK_1M = Workload("chunked_prefill_1m_8k", 1, 8192, 1040384, 1048576, 2048, "FSSS", 64,
                    128, "fp8", 16, 576, 512)

WORKLOADS = {w.name: w for w in (TINY_L1K, L16K, L128K, DECODE_B32, CHUNK_1M)}

# hidden width feeding the indexer projection (GLM-5.2 configuration)
D_HIDDEN = 6144


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _normal(shape, std, gen, device, dtype, chunk_rows=1 << 14):
    """N(0, std^2) drawn in fp32 and rounded to ``dtype``; chunked along dim 0
    so a multi-GB tensor never needs a full fp32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(-1, 1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        t = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        flat[r0:r1].copy_(t)
    return out


def _ints(shape, lo, hi, gen, device, dtype):
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device,
                         dtype=torch.int32).to(dtype)


def fp8_rows(k32: torch.Tensor):
    """Per-row e4m3fn codes and fp32 scales for fp32 rows ``k32[..., d]``."""
    amax = k32.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (k32 / scale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale.squeeze(-1).contiguous()


def indexer_keys(w: Workload, device, layer: int = 0):
    """Indexer key cache for one full layer: returns (keys, scale).

    keys: [B, cap, d] bf16, or uint8 e4m3fn codes; scale: [B, cap] fp32 or None.
    """
    shape = (w.batch, w.cap, w.ix_dim)
    g = _gen(device, w.seed, w.name, "ix_k", layer)
    if w.mode == "exact":
        if w.key_dtype == "bf16":
            return _ints(shape, -8, 8, g, device, torch.bfloat16), None
        codes = _ints(shape, -8, 8, g, device, torch.float32).to(torch.float8_e4m3fn)
        return codes.view(torch.uint8), torch.ones(shape[:2], dtype=torch.float32,
                                                    device=device)
    if w.key_dtype == "bf16":
        return _normal(shape, 1.0 / math.sqrt(w.ix_dim), g, device, torch.bfloat16), None
    codes = torch.empty(shape, dtype=torch.uint8, device=device)
    scale = torch.empty(shape[:2], dtype=torch.float32, device=device)
    rows = 1 << 15
    for b in range(w.batch):
        for r0 in range(0, w.cap, rows):
            r1 = min(w.cap, r0 + rows)
            k32 = torch.randn((r1 - r0, w.ix_dim), generator=g, device=device,
                              dtype=torch.float32)
            c, s = fp8_rows(k32)
            codes[b, r0:r1] = c.view(torch.uint8)
            scale[b, r0:r1] = s
    return codes, scale


def new_key_rows(w: Workload, device, step: int = 0, layer: int = 0):
    """fp32 indexer key rows [B, 1, d] of the token a decode step appends
    (N(0,1), seeded per step)."""
    g = _gen(device, w.seed, w.name, "ix_knew", layer, step)
    return torch.randn((w.batch, 1, w.ix_dim), generator=g, device=device, dtype=torch.float32)


def indexer_queries(w: Workload, device, layer: int = 0, step: int = 0):
    """Indexer queries [B, n_q, H, d] bf16 and head weights [B, n_q, H] fp32."""
    g = _gen(device, w.seed, w.name, "ix_q", layer, step)
    qs = (w.batch, w.n_q, w.ix_heads, w.ix_dim)
    ws = (w.batch, w.n_q, w.ix_heads)
    if w.mode == "exact":
        q = _ints(qs, -8, 8, g, device, torch.bfloat16)
        e = torch.randint(0, 3, ws, generator=g, device=device, dtype=torch.int32)
        wt = torch.pow(2.0, e.to(torch.float32))
        return q, wt
    q = _normal(qs, 1.0 / math.sqrt(w.ix_dim), g, device, torch.bfloat16)
    wt = torch.randn(ws, generator=g, device=device, dtype=torch.float32)
    return q, wt


def indexer_queries_fp8(w: Workload, device, layer: int = 0, step: int = 0):
    """fp8 indexer queries: (codes [B, n_q, H, d] uint8 e4m3fn, q_scale
    [B, n_q, H] fp32, head weights [B, n_q, H] fp32)."""
    g = _gen(device, w.seed, w.name, "ix_q8", layer, step)
    qs = (w.batch, w.n_q, w.ix_heads, w.ix_dim)
    ws = (w.batch, w.n_q, w.ix_heads)
    if w.mode == "exact":
        codes = _ints(qs, -8, 8, g, device, torch.float32).to(torch.float8_e4m3fn)
        e = torch.randint(-1, 2, ws, generator=g, device=device, dtype=torch.int32)
        q_scale = torch.pow(2.0, e.to(torch.float32))
        e = torch.randint(0, 3, ws, generator=g, device=device, dtype=torch.int32)
        wt = torch.pow(2.0, e.to(torch.float32))
        return codes.view(torch.uint8), q_scale, wt
    q32 = torch.randn(qs, generator=g, device=device, dtype=torch.float32) / math.sqrt(w.ix_dim)
    codes, q_scale = fp8_rows(q32)
    wt = torch.randn(ws, generator=g, device=device, dtype=torch.float32)
    return codes.view(torch.uint8), q_scale, wt


def attn_queries(w: Workload, device, layer: int, step: int = 0):
    """Attention queries [B, n_q, Hq, D] bf16 ~ N(0, 1)."""
    g = _gen(device, w.seed, w.name, "attn_q", layer, step)
    return _normal((w.batch, w.n_q, w.q_heads, w.d_qk), 1.0, g, device, torch.bfloat16)


def latent_kv(w: Workload, device, layer: int):
    """Latent KV cache [B, cap, D] bf16 ~ N(0, 1); V is its first d_v dims."""
    g = _gen(device, w.seed, w.name, "kv", layer)
    return _normal((w.batch, w.cap, w.d_qk), 1.0, g, device, torch.bfloat16)


def sample_rows(w: Workload, n: int = 64, seed: int = 0):
    """Query rows sampled for full-size checks: first and last rows, the rows
    whose candidate count is k-1, k and k+1 (when they exist), and a seeded
    uniform draw for the rest.  Returned sorted and unique."""
    rows = {0, w.n_q - 1}
    for nt in (w.k - 1, w.k, w.k + 1):
        t = nt - 1 - w.q_start
        if 0 <= t < w.n_q:
            rows.add(t)
    g = torch.Generator().manual_seed(_seed(seed, w.name, "rows"))
    extra = torch.randint(0, w.n_q, (4 * n,), generator=g).tolist()
    for t in extra:
        if len(rows) >= min(n, w.n_q):
            break
        rows.add(int(t))
    return sorted(rows)


def projection_inputs(w: Workload, device, layer: int = 0, d_in: int = D_HIDDEN):
    """Hidden-state rows [B * n_q, d_in] and the stacked indexer projection
    weight [H*d + H, d_in] (q_I rows first, then one row per head weight),
    both bf16."""
    rows, n = w.batch * w.n_q, w.ix_heads * w.ix_dim + w.ix_heads
    gx = _gen(device, w.seed, w.name, "proj_x", layer)
    gw = _gen(device, w.seed, w.name, "proj_w", layer)
    if w.mode == "exact":
        return (_ints((rows, d_in), -8, 8, gx, device, torch.bfloat16),
                _ints((n, d_in), -8, 8, gw, device, torch.bfloat16))
    return (_normal((rows, d_in), 1.0, gx, device, torch.bfloat16),
            _normal((n, d_in), 1.0 / math.sqrt(d_in), gw, device, torch.bfloat16))
