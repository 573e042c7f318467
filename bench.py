"""Benchmark of the DSA layer group under the IndexShare schedule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config l128k|l16k|tiny|chunk1m|decode]

A step is one pass of the whole hot path over one synthetic batch: for the
default (headline) workload that is L = 131072 query rows through 8 layers
arranged as two full+shared+shared+shared groups -- the indexer + streaming
top-k on the 2 full layers and sparse attention on all 8.  Inputs are
generated on the device before timing starts.  Prints one JSON line.

    python bench.py --op indexer|attention [--steps K] [--warmup W]

times one op of the workload's first layer alone (for profilers).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBPS = 8000.0

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_attn_prefill_l128k.json")
ATTN_SOURCE = os.path.join(ROOT, "long_context_sparse_ix_amd", "csrc", "sparse_attn.hip")
CAL_BYTES = 1 << 30            # plain device copy used to scale the HBM byte counters

CONFIGS = {"tiny": "tiny_l1k_exact", "l16k": "prefill_l16k", "l128k": "prefill_l128k_2groups",
           "decode": "decode_b32_ctx200k", "chunk1m": "chunked_prefill_1m_8k"}


def causal_pairs(w, n_rows=None):
    """sum over query rows of the candidate count p+1 (keys each row scores)."""
    n = w.n_q if n_rows is None else n_rows
    a = w.q_start + 1
    return w.batch * (n * a + n * (n - 1) // 2)


def gathered_rows(w):
    """sum over query rows of min(k, p+1): latent rows each row attends over."""
    tot = 0
    k = w.k
    lo, hi = w.q_start + 1, w.q_start + w.n_q          # candidate counts of first/last row
    if hi <= k:
        tot = (lo + hi) * w.n_q // 2
    elif lo >= k:
        tot = k * w.n_q
    else:
        m = k - lo + 1                                   # rows with count <= k
        tot = (lo + k) * m // 2 + k * (w.n_q - m)
    return w.batch * tot


class Inputs:
    """Device inputs for every layer of the workload (generated, then kept resident)."""

    def __init__(self, w, synth, torch, all_full: bool, step: int = 0):
        self.w = w
        dev = "cuda"
        n = w.n_layers
        self.ix = []
        for l in range(n):
            if w.roles[l] == "F" or all_full:
                q, wt = synth.indexer_queries(w, dev, l, step)
                keys, scale = synth.indexer_keys(w, dev, l)
                self.ix.append(dict(q=q, w=wt, keys=keys, k_scale=scale))
            else:
                self.ix.append(None)
        self.attn = []
        for l in range(n):
            self.attn.append(dict(q=synth.attn_queries(w, dev, l, step), kv=synth.latent_kv(w, dev, l),
                                  out=torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16,
                                                  device=dev)))
        self.idx_fs = torch.empty((w.roles.count("F"), w.batch, w.n_q, w.k), dtype=torch.int32, device=dev)
        self.idx_ff = torch.empty((n, w.batch, w.n_q, w.k), dtype=torch.int32, device=dev) if all_full else None


def source_sha(path):
    """SHA-256 of a kernel source's code: comments and blank space removed, so
    an edit to the comments keeps counters taken on the same code valid."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def attention_bytes(w):
    """Algorithmic bytes of one sparse-attention launch: gathered latent rows
    plus every row's Q, O and index words."""
    rows = w.batch * w.n_q
    return (gathered_rows(w) * w.d_qk * 2 + rows * w.q_heads * (w.d_qk + w.d_v) * 2 + rows * w.k * 4)


def load_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing, was taken on another version of the kernel, or
    on another workload (the counters were taken at one size only)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha(ATTN_SOURCE) or t.get("workload") != workload:
        return None
    return t


def write_traffic(fetch_dir, write_dir, command):
    """Turns two rocprofv3 --pmc runs of `bench.py --copy-calibration` (one
    with FETCH_SIZE, one with WRITE_SIZE) into the traffic summary: the
    attention kernel's KiB per dispatch, scaled by CAL_BYTES over what the
    same counter reads for the calibration copy."""
    def per_kernel(d, counter):
        path = os.path.join(d, "pmc_counter_collection.csv")
        att, cal = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if "sparse_attn_kernel" in r["Kernel_Name"]:
                    att.append(v)
                elif "copyBuffer" in r["Kernel_Name"]:
                    cal.append(v)
        cal = sorted(cal)[-4:]                     # the CAL_BYTES copies are the largest
        return sum(att) / len(att), sum(cal) / len(cal), len(att)
    fa, fc, n = per_kernel(fetch_dir, "FETCH_SIZE")
    wa, wc, _ = per_kernel(write_dir, "WRITE_SIZE")
    f_fac, w_fac = CAL_BYTES / (fc * 1024), CAL_BYTES / (wc * 1024)
    out = {"kernel": "sparse_attn_kernel", "workload": "prefill_l128k_2groups", "dispatches": n,
           "fetch_kib_per_dispatch": fa, "write_kib_per_dispatch": wa,
           "calibration": {"copy_bytes": CAL_BYTES, "fetch_kib": fc, "write_kib": wc,
                           "fetch_factor": f_fac, "write_factor": w_fac},
           "hbm_bytes_per_launch": fa * 1024 * f_fac + wa * 1024 * w_fac,
           "source_sha256": source_sha(ATTN_SOURCE),
           "source_sha256_of": "sparse_attn.hip with comments and blank space removed (the code the counters were taken on)",
           "command": command}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def event_time(torch, fn, reps):
    """Average ms of fn() over reps runs, timed with events on the current
    stream (the stream every library call enqueues on)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_baseline(w, inp, torch, rows, np_threads):
    """Time the CPU oracle on the sampled rows of this workload and
    extrapolate to the whole step with the per-row cost model (indexer and
    top-k ~ candidates per row, attention ~ min(k, candidates))."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import dsa_oracle as O

    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    host = {}
    for l in range(w.n_layers):
        a = inp.attn[l]
        host[l] = dict(Q=bits(a["q"][:, rows]), KV=bits(a["kv"]))
        if w.roles[l] == "F":
            e = inp.ix[l]
            kb = bits(e["keys"]) if e["keys"].dtype == torch.bfloat16 else e["keys"].view(torch.uint8).cpu().numpy()
            host[l].update(q=bits(e["q"][:, rows]), w=e["w"][:, rows].cpu().numpy(), keys=kb,
                           kd="bf16" if e["keys"].dtype == torch.bfloat16 else "fp8",
                           scale=None if e["k_scale"] is None else e["k_scale"].cpu().numpy())
    sm = 1.0 / math.sqrt(w.d_qk)
    t_ix = t_at = 0.0
    idx_oracle, outs = [], []
    cur = None
    with threadpool_limits(limits=np_threads):
        for l in range(w.n_layers):
            h = host[l]
            if w.roles[l] == "F":
                t0 = time.perf_counter()
                # rows are passed with their absolute positions via q_start + t
                res = np.stack([O.indexer_topk(h["q"][:, i:i + 1], h["w"][:, i:i + 1], h["keys"], h["kd"],
                                               h["scale"], w.q_start + t, w.kv_len, w.k)[:, 0]
                                for i, t in enumerate(rows)], axis=1)
                t_ix += time.perf_counter() - t0
                idx_oracle.append(res)
                cur = inp.idx_fs[len(idx_oracle) - 1][:, rows].cpu().numpy()   # attention is checked given the GPU's indices
            t0 = time.perf_counter()
            o, _ = O.sparse_attention(h["Q"], h["KV"], cur, w.kv_len, sm, w.d_v)
            t_at += time.perf_counter() - t0
            outs.append(o)
    n_f = w.roles.count("F")
    samp_pairs = sum(w.q_start + t + 1 for t in rows) * w.batch
    samp_rows = sum(min(w.k, w.q_start + t + 1) for t in rows) * w.batch
    full_ix = t_ix * causal_pairs(w) / samp_pairs
    full_at = t_at * gathered_rows(w) / samp_rows
    return dict(t_ix=t_ix, t_at=t_at, full_s=full_ix + full_at, idx=idx_oracle, O=outs,
                n_f=n_f, samp_rows=len(rows))


def sampled_parity(w, inp, rows, cb, torch):
    """GPU vs oracle on the sampled rows: index-set overlap per full layer and
    max-abs error of every layer's output given the GPU's indices."""
    import numpy as np

    ovl = []
    for f, ref in enumerate(cb["idx"]):
        got = inp.idx_fs[f][:, rows].cpu().numpy()
        inter = tot = 0
        for g, r in zip(got.reshape(-1, w.k), ref.reshape(-1, w.k)):
            sr = set(r[r >= 0].tolist())
            inter += len(set(g[g >= 0].tolist()) & sr)
            tot += len(sr)
        ovl.append(inter / max(tot, 1))
    err = max(float(np.abs(inp.attn[l]["out"][:, rows].float().cpu().numpy() - cb["O"][l]).max())
              for l in range(w.n_layers))
    return {"rows": len(rows), "idx_overlap_min": min(ovl), "attn_max_abs_err": err,
            "ok": min(ovl) >= 0.999 and err <= 2e-2}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 3; decode: 60, so that with the warmup the 64 decode "
                         "steps of the workload run)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 1; decode: 4)")
    ap.add_argument("--config", default="l128k", choices=sorted(CONFIGS))
    ap.add_argument("--kernel-reps", type=int, default=3)
    ap.add_argument("--sample-rows", type=int, default=0,
                    help="rows checked against the oracle and timed on the CPU (0: 48, fewer for "
                         "rows of more than 512K candidates so the CPU leg stays near half a minute)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-full", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, copy a 1 GiB device buffer 4 times (HBM counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the attention traffic summary from two rocprofv3 --pmc output dirs")
    ap.add_argument("--traffic-command", default="", help="command recorded with --write-traffic")
    ap.add_argument("--op", choices=["indexer", "attention"],
                    help="time one op of the workload's first layer alone (warmup + steps launches), for profiling")
    args = ap.parse_args(argv)
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.traffic_command)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the DSA group path runs on exactly one GPU; it has no multi-GPU "
                          "mode, so --gpus must be 1"}))
        return 2

    import numpy as np
    import torch

    import ix_synth as synth
    import long_context_sparse_ix_amd as ix

    if not os.path.exists(ix.LIB_PATH):
        from long_context_sparse_ix_amd import build
        build.build()
    ix.load()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[CONFIGS[args.config]]
    if w.decode_steps and not args.op:
        args.warmup = 4 if args.warmup is None else args.warmup
        args.steps = w.decode_steps - args.warmup if args.steps is None else args.steps
    args.warmup = 1 if args.warmup is None else args.warmup
    args.steps = 3 if args.steps is None else args.steps
    if args.op:
        return bench_op(args, w, torch, synth, ix)
    if w.decode_steps:
        return bench_decode(args, w, torch, synth, ix)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    log(f"workload {w.name}: generating inputs")
    inp = Inputs(w, synth, torch, all_full=not args.no_all_full)
    torch.cuda.synchronize()
    fs_mask = w.f_mask

    def run_group(mask, idx):
        ix.ix_group_forward(inp.ix, inp.attn, mask, idx, q_start=w.q_start, kv_len=w.kv_len)

    log("warmup")
    for _ in range(args.warmup):
        run_group(fs_mask, inp.idx_fs)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        run_group(fs_mask, inp.idx_fs)
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    n_groups = w.n_layers // 4
    tok_per_group = w.batch * w.n_q / (ms_step / n_groups / 1e3)

    log("per-kernel timing")
    e = inp.ix[0]
    idx0 = inp.idx_fs[0]
    ix_ms = event_time(torch, lambda: ix.ix_indexer_topk(e["q"], e["w"], e["keys"], idx0, k_scale=e["k_scale"],
                                                         q_start=w.q_start, kv_len=w.kv_len), args.kernel_reps)
    a = inp.attn[1]
    at_ms = event_time(torch, lambda: ix.ix_sparse_attn(a["q"], a["kv"], idx0, a["out"], q_start=w.q_start,
                                                        kv_len=w.kv_len), args.kernel_reps)
    ix_flop = causal_pairs(w) * 2 * w.ix_heads * w.ix_dim
    ix_tflops = ix_flop / (ix_ms / 1e3) / 1e12
    g_rows = gathered_rows(w)
    at_bytes = attention_bytes(w)
    at_gbps = at_bytes / (at_ms / 1e3) / 1e9
    at_flop = g_rows * w.q_heads * 2 * (w.d_qk + w.d_v)

    # standalone row top-k over materialised fp32 rows at the decode shape
    # (32 rows of 200,001 scores): HBM fraction on one read of the rows
    g = torch.Generator(device="cuda").manual_seed(0)
    dk = synth.DECODE_B32
    tk_scores = torch.randn((dk.batch, 1, dk.kv_len), generator=g, device="cuda")
    tk_idx = torch.empty((dk.batch, 1, dk.k), dtype=torch.int32, device="cuda")
    tk_ms = event_time(torch, lambda: ix.ix_topk_scores(tk_scores, tk_idx, q_start=dk.q_start, kv_len=dk.kv_len),
                       max(args.kernel_reps, 10))
    tk_bytes = dk.batch * (4 * dk.kv_len + 4 * dk.k)
    del tk_scores

    # overlap of the two full layers' index buffers (the adjacent-layer
    # overlap that makes reuse work), when the workload has two full layers
    overlap = None
    if inp.idx_fs.shape[0] >= 2:
        cnt = ix.ix_index_overlap(inp.idx_fs[0], inp.idx_fs[1])
        ov_ms = event_time(torch, lambda: ix.ix_index_overlap(inp.idx_fs[0], inp.idx_fs[1], cnt), 5)
        valid = (inp.idx_fs[0] >= 0).sum(dim=-1).clamp(min=1)
        overlap = {"layers": "first vs second full layer", "mean_fraction": float((cnt.float() / valid).mean()),
                   "us": ov_ms * 1e3, "rows_per_s": w.batch * w.n_q / (ov_ms / 1e3),
                   "note": "independent synthetic layers: about k / candidates expected"}

    allf_ms = None
    if not args.no_all_full:
        log("all-full baseline")
        allf_mask = (1 << w.n_layers) - 1
        allf_ms = event_time(torch, lambda: run_group(allf_mask, inp.idx_ff), 1)
        # all-F baseline re-ran the F layers' slots; restore the F+3S indices
        run_group(fs_mask, inp.idx_fs)
        torch.cuda.synchronize()

    tr = load_traffic(w.name)
    traffic_bytes = None if tr is None else tr["hbm_bytes_per_launch"]

    n_sample = args.sample_rows
    if n_sample <= 0:   # the oracle costs about 2 s per row at 1M candidates
        n_sample = 48 if w.kv_len <= 512 * 1024 else 12
    rows = synth.sample_rows(w, n_sample)
    result_cpu, parity = None, None
    if not args.no_cpu_baseline:
        log(f"CPU oracle on {len(rows)} sampled rows")
        cores = min(16, len(os.sched_getaffinity(0)))
        cb = cpu_baseline(w, inp, torch, rows, cores)
        n_tokens = w.batch * w.n_q
        cpu_tok = n_tokens / (cb["full_s"] / n_groups)
        result_cpu = {"value": cpu_tok, "unit": "tokens/s per group", "cores": cores, "kind": "oracle",
                      "sample": f"{len(rows)} query rows of {w.n_q} (all {w.n_layers} layers; indexer on "
                                f"{cb['n_f']} full layers) timed {cb['t_ix'] + cb['t_at']:.1f}s, extrapolated "
                                f"by rows' candidate counts (indexer) and min(k, candidates) (attention)"}
        parity = sampled_parity(w, inp, rows, cb, torch)

    out = {
        "metric": "prefill tokens/s per 4-layer F,S,S,S group at L=128K; indexer TFLOP/s; HBM %"
        if w.name == synth.L128K.name else f"prefill tokens/s per 4-layer F,S,S,S group ({w.name})",
        "value": tok_per_group, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, on device)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.kv_len, "query_rows": w.n_q,
                   "q_start": w.q_start, "roles": w.roles, "k": w.k,
                   "indexer": f"{w.ix_heads} heads x {w.ix_dim}, {w.key_dtype} keys",
                   "attention": f"{w.q_heads} heads over 1 latent head {w.d_qk} (V = first {w.d_v})"},
        "roofline": {"bound": "hbm", "achieved": at_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": at_gbps / PEAK_HBM_GBPS, "traffic": traffic_bytes,
                     "kernel": "sparse_attn_kernel: (gathered latent rows + Q + O + idx bytes) per launch "
                               "/ launch time; traffic = HBM bytes per launch from FETCH_SIZE + WRITE_SIZE",
                     "algorithmic_bytes": at_bytes},
        "indexer": {"ms": ix_ms, "tflops": ix_tflops, "frac_bf16_peak": ix_tflops / PEAK_BF16_TFLOPS,
                    "frac_fp8_peak": ix_tflops / PEAK_FP8_TFLOPS, "flop": ix_flop,
                    "note": "fused score + streaming top-k, incl. staging the keys as bf16 (fp8 widened exactly)"},
        "attention": {"ms_per_layer": at_ms, "tokens_per_s": w.batch * w.n_q / (at_ms / 1e3),
                      "gathered_GBps": at_gbps, "frac_hbm_peak": at_gbps / PEAK_HBM_GBPS,
                      "tflops": at_flop / (at_ms / 1e3) / 1e12},
        "topk_standalone": {"workload": "32 rows x 200,001 fp32 scores, k=2048", "us": tk_ms * 1e3,
                            "rows_per_s": dk.batch / (tk_ms / 1e3),
                            "frac_hbm_peak": tk_bytes / (tk_ms / 1e3) / 1e9 / PEAK_HBM_GBPS},
        "index_overlap": overlap,
        "group": {"ms_fsss": ms_step / n_groups, "ms_all_full": None if allf_ms is None else allf_ms / n_groups,
                  "speedup_vs_all_full": None if allf_ms is None else allf_ms / ms_step},
        "cpu_baseline": result_cpu,
        "parity": parity,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        src = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
    return 0


def bench_op(args, w, torch, synth, ix):
    """One op of the first layer, launched warmup + steps times: the indexer
    (+ fused top-k) or the sparse attention over that indexer's positions."""
    dev = "cuda"
    q, wt = synth.indexer_queries(w, dev, 0)
    keys, scale = synth.indexer_keys(w, dev, 0)
    idx = torch.empty((w.batch, w.n_q, w.k), dtype=torch.int32, device=dev)
    run_ix = lambda: ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len)
    fn = run_ix
    if args.op == "attention":
        run_ix()
        del q, wt, keys, scale
        aq = synth.attn_queries(w, dev, 0)
        kv = synth.latent_kv(w, dev, 0)
        out = torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device=dev)
        fn = lambda: ix.ix_sparse_attn(aq, kv, idx, out, q_start=w.q_start, kv_len=w.kv_len)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    ms = event_time(torch, fn, args.steps) if args.steps > 0 else None
    print(json.dumps({"op": args.op, "workload": w.name, "launches": args.warmup + args.steps + 1,
                      "ms_per_launch": ms}), flush=True)
    if args.copy_calibration:
        src = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
    return 0


def decode_oracle_leg(w, torch, keys, scale, kvs, step_inputs, last, j, log, n_seq=12):
    """The CPU oracle on n_seq sequences of decode step j (indexer over the
    whole cache, then the four layers' attention over the GPU's positions),
    timed and extrapolated to the batch; parity of those sequences."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import dsa_oracle as O

    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    seqs = list(range(0, w.batch, max(1, w.batch // n_seq)))[:n_seq]
    q_start, kv_len = w.q_start + j, w.kv_len + j
    ixl, att = step_inputs
    ixe = ixl[0]                                   # the full layer's indexer inputs
    sel = torch.tensor(seqs, device=keys.device)
    h_q, h_w = bits(ixe["q"][sel]), ixe["w"][sel].cpu().numpy()
    h_k, h_s = keys[sel, :kv_len].contiguous().cpu().numpy(), scale[sel, :kv_len].cpu().numpy()
    gpu_idx = last["idx"][sel]                                      # [S, 1, k]
    # attention inputs: only the selected latent rows leave the device
    gidx = gpu_idx.clamp(min=0).long()
    att_in = []
    for l in range(4):
        kvg = torch.stack([kvs[l][b][gidx[i, 0]] for i, b in enumerate(seqs)])   # [S, k, D]
        att_in.append((bits(att[l]["q"][sel]), bits(kvg)))
    slot = torch.where(gpu_idx >= 0, torch.arange(w.k, device=keys.device).view(1, 1, -1),
                       torch.full_like(gpu_idx, -1)).cpu().numpy().astype(np.int32)
    cores = min(16, len(os.sched_getaffinity(0)))
    log(f"CPU oracle on {len(seqs)} sequences of decode step {j}")
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        ref_idx = O.indexer_topk(h_q, h_w, h_k, "fp8", h_s, q_start, kv_len, w.k)
        t_ix = time.perf_counter() - t0
        t0 = time.perf_counter()
        ref_o = [O.sparse_attention(qb, kvb, slot, w.k, 1.0 / math.sqrt(w.d_qk), w.d_v)[0] for qb, kvb in att_in]
        t_at = time.perf_counter() - t0
    got = gpu_idx.cpu().numpy()
    inter = tot = 0
    for g, r in zip(got.reshape(-1, w.k), ref_idx.reshape(-1, w.k)):
        sr = set(r[r >= 0].tolist())
        inter += len(set(g[g >= 0].tolist()) & sr)
        tot += len(sr)
    ovl = inter / max(tot, 1)
    err = max(float(np.abs(last["outs"][l][sel].float().cpu().numpy() - ref_o[l]).max()) for l in range(4))
    step_s = (t_ix + t_at) * w.batch / len(seqs)
    cpu = {"value": w.batch / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{len(seqs)} of {w.batch} sequences of one decode step (indexer over {kv_len:,} keys, "
                     f"4 layers of attention) timed {t_ix + t_at:.1f}s, extrapolated to the batch"}
    parity = {"sequences": len(seqs), "idx_overlap": ovl, "attn_max_abs_err": err,
              "ok": ovl >= 0.999 and err <= 2e-2}
    return cpu, parity


def bench_decode(args, w, torch, synth, ix):
    """Decode: each step appends one token to each of B sequences and runs one
    full+3 shared layer group for the new query rows."""
    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    log(f"workload {w.name}: generating caches")
    dev = "cuda"
    keys, scale = synth.indexer_keys(w, dev, 0)
    kvs = [synth.latent_kv(w, dev, l) for l in range(4)]
    total = args.warmup + args.steps
    steps = []
    for j in range(total):
        q, wt = synth.indexer_queries(w, dev, 0, j)
        att = [dict(q=synth.attn_queries(w, dev, l, j), kv=kvs[l],
                    out=torch.empty((w.batch, 1, w.q_heads, w.d_v), dtype=torch.bfloat16, device=dev))
               for l in range(4)]
        steps.append(([dict(q=q, w=wt, keys=keys, k_scale=scale), None, None, None], att))
    idx = torch.empty((1, w.batch, 1, w.k), dtype=torch.int32, device=dev)
    new_keys = [synth.new_key_rows(w, dev, j) for j in range(total)]

    def run(j, mask=1):
        # the new token's indexer key is quantized into the fp8 cache at its
        # position, then the layer group runs for the new query rows
        ix.ix_append_keys(new_keys[j], keys, scale, w.q_start + j)
        ixl, att = steps[j]
        if mask != 1:
            ixl = [ixl[0]] * 4
        ix.ix_group_forward(ixl, att, mask, idx if mask == 1 else idx_ff, q_start=w.q_start + j,
                            kv_len=w.kv_len + j)

    idx_ff = torch.empty((4, w.batch, 1, w.k), dtype=torch.int32, device=dev)
    for j in range(args.warmup):
        run(j)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for j in range(args.warmup, total):
        run(j)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the last timed step's results, for the oracle leg below (later runs overwrite them)
    j_last = total - 1
    last = dict(idx=idx[0].clone(), outs=[a["out"].clone() for a in steps[j_last][1]])
    allf = event_time(torch, lambda: run(args.warmup, mask=0xF), 2)
    key_bytes = w.batch * (w.kv_len + args.warmup) * (w.ix_dim + 4)
    app_ms = event_time(torch, lambda: ix.ix_append_keys(new_keys[0], keys, scale, w.q_start), 20)

    # sequences of different lengths: the same group step with contexts spread
    # evenly over [context/2, context] (per-sequence starts read on the device)
    lo = w.q_start // 2
    starts = torch.linspace(lo, w.q_start, w.batch, device=dev).round().to(torch.int64)
    ixl0, att0 = steps[args.warmup]
    varlen_ms = event_time(torch, lambda: ix.ix_group_forward(ixl0, att0, 1, idx, q_start=w.q_start, kv_len=w.kv_len,
                                                              seq_q_start=starts), 5)
    varlen = {"contexts": f"{w.batch} sequences, {lo + 1:,}..{w.q_start + 1:,} keys evenly spaced",
              "ms_fsss": varlen_ms, "tokens_per_s": w.batch / (varlen_ms / 1e3)}

    # MTP draft steps on one layer: the first step selects, the later steps
    # attend over its positions in the same cache; against every step
    # selecting anew at its own position
    n_draft = 5
    e = ixl0[0]
    kv0 = kvs[0]
    dq = [steps[args.warmup + (j % args.steps)][1][0]["q"] for j in range(n_draft)]
    d_out = torch.empty((w.batch, 1, w.q_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    d_idx = torch.empty((w.batch, 1, w.k), dtype=torch.int32, device=dev)

    def draft(reuse):
        for j in range(n_draft):
            if j == 0 or not reuse:
                ix.ix_indexer_topk(e["q"], e["w"], keys, d_idx, k_scale=scale, q_start=w.q_start + j,
                                   kv_len=w.kv_len + j)
            ix.ix_sparse_attn(dq[j], kv0, d_idx, d_out, q_start=w.q_start, kv_len=w.kv_len + n_draft)

    reuse_ms = event_time(torch, lambda: draft(True), 5)
    reselect_ms = event_time(torch, lambda: draft(False), 5)
    mtp = {"draft_steps": n_draft, "ms_reuse": reuse_ms, "ms_reselect_every_step": reselect_ms,
           "speedup": reselect_ms / reuse_ms,
           "note": "one MTP layer, B sequences: the indexer + top-k once, then attention per step"}
    # dominant op: the full layer's indexer + top-k (score kernel streaming the
    # fp8 keys, then the one-pass merge), 58-60% of the step
    ixe = steps[j_last][0][0]
    ix_idx = torch.empty((w.batch, 1, w.k), dtype=torch.int32, device=dev)
    ix_ms = event_time(torch, lambda: ix.ix_indexer_topk(ixe["q"], ixe["w"], keys, ix_idx, k_scale=scale,
                                                         q_start=w.q_start + j_last, kv_len=w.kv_len + j_last), 20)
    ix_bytes = w.batch * (w.kv_len + j_last) * (w.ix_dim + 4 + 4)
    ix_gbps = ix_bytes / (ix_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": ix_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": ix_gbps / PEAK_HBM_GBPS, "traffic": None,
                "kernel": "ix_indexer_topk per call (indexer_scores_kernel + tk_merge_kernel): fp8 key codes + "
                          "scale read and one fp32 score written per (row, key)",
                "algorithmic_bytes": ix_bytes}

    result_cpu, parity = None, None
    if not args.no_cpu_baseline:
        result_cpu, parity = decode_oracle_leg(w, torch, keys, scale, kvs, steps[j_last], last, j_last, log)
    out = {"metric": "decode tokens/s (B=32, 200K context, one F,S,S,S group per step)",
           "value": w.batch / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, on device)",
           "config": {"workload": w.name, "batch": w.batch, "context": w.kv_len, "k": w.k},
           "step": "quantize+append the new token's indexer key into the fp8 cache, then the F,S,S,S group",
           "roofline": roofline, "cpu_baseline": result_cpu, "parity": parity,
           "append_keys_us": app_ms * 1e3,
           "group": {"ms_fsss": ms, "ms_all_full": allf, "speedup_vs_all_full": allf / ms},
           "varlen": varlen, "mtp_draft": mtp,
           "indexer_key_GBps_lower_bound": key_bytes / (ms / 1e3) / 1e9}
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
