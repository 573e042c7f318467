"""Benchmark of the DSA layer group under the IndexShare schedule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config l128k|l16k|tiny|chunk1m|decode]

A step is one pass of the whole hot path over one synthetic batch: for the
default (headline) workload that is L = 131072 query rows through 8 layers
arranged as two full+shared+shared+shared groups -- the indexer + streaming
top-k on the 2 full layers and sparse attention on all 8.  Inputs are
generated on the device before timing starts.  Prints one JSON line.

    python bench.py --op indexer|argmax|attention|project|topk [--fp8-queries] [--config ...] [--steps K] [--warmup W]

times one op of the workload's first layer alone (for profilers): the indexer
with its streaming top-k, the same score stream with a running maximum
instead of the top-k (ix_indexer_argmax), the sparse attention, the
indexer projection, or the row top-k alone over 32 rows of 200,001 fp32
scores (ix_topk_scores); --fp8-queries poses the indexer's queries as e4m3fn
codes with a per-(row, head) scale.

    python bench.py --write-traffic FETCH_DIR WRITE_DIR --traffic-op indexer|attention [--config ...]

turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of an --op run
with --copy-calibration into the committed traffic summary of that kernel.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2
PEAK_HBM_GBPS = 8000.0

CSRC = os.path.join(ROOT, "long_context_sparse_ix_amd", "csrc")
CAL_BYTES = 1 << 30            # plain device copy used to scale the HBM byte counters
# kernels whose HBM traffic is summarised under profiles/: op -> (kernel name, source file)
TRAFFIC_OPS = {"indexer": ("fused_indexer_topk_kernel", "indexer_fused.hip"),
               "attention": ("sparse_attn_kernel", "sparse_attn.hip")}

CONFIGS = {"tiny": "tiny_l1k_exact", "l16k": "prefill_l16k", "l128k": "prefill_l128k_2groups",
           "decode": "decode_b32_ctx200k", "chunk1m": "chunked_prefill_1m_8k"}

# CPU share of one GPU on the benchmark hosts: oracle worker processes are
# capped at this (or at the cores the process may run on, if fewer)
HOST_CPU_SHARE = 16


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


# ------------------------------------------------------------ HBM traffic --
def source_sha(path):
    """SHA-256 of a kernel source's code: comments and blank space removed, so
    an edit to the comments keeps counters taken on the same code valid."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def traffic_path(op, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{TRAFFIC_OPS[op][0]}_{workload}.json")


def load_traffic(op, workload):
    """HBM bytes per launch of op's kernel on this workload from the committed
    counter summary, or None when there is none or it was taken on another
    version of the kernel's source."""
    try:
        with open(traffic_path(op, workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha(os.path.join(CSRC, TRAFFIC_OPS[op][1])):
        return None
    return t


def write_traffic(op, workload, fetch_dir, write_dir, command):
    """Turns two rocprofv3 --pmc runs of `bench.py --op <op> --copy-calibration`
    (one with FETCH_SIZE, one with WRITE_SIZE) into the traffic summary: the
    kernel's KiB per dispatch, each counter scaled by CAL_BYTES over what it
    reads for the calibration copy."""
    kernel, src = TRAFFIC_OPS[op]

    def per_kernel(d, counter):
        path = os.path.join(d, "pmc_counter_collection.csv")
        if not os.path.exists(path):     # rocprofv3 may put the csv under a host/pid subfolder
            hits = [os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs
                    if f.endswith("counter_collection.csv")]
            path = hits[0]
        ker, cal = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if kernel in r["Kernel_Name"]:
                    ker.append(v)
                elif "copyBuffer" in r["Kernel_Name"]:
                    cal.append(v)
        cal = sorted(cal)[-4:]                     # the CAL_BYTES copies are the largest
        return sum(ker) / len(ker), sum(cal) / len(cal), len(ker)

    fa, fc, n = per_kernel(fetch_dir, "FETCH_SIZE")
    wa, wc, _ = per_kernel(write_dir, "WRITE_SIZE")
    f_fac, w_fac = CAL_BYTES / (fc * 1024), CAL_BYTES / (wc * 1024)
    out = {"kernel": kernel, "workload": workload, "dispatches": n,
           "fetch_kib_per_dispatch": fa, "write_kib_per_dispatch": wa,
           "calibration": {"copy_bytes": CAL_BYTES, "fetch_kib": fc, "write_kib": wc,
                           "fetch_factor": f_fac, "write_factor": w_fac},
           "read_bytes_per_launch": fa * 1024 * f_fac, "write_bytes_per_launch": wa * 1024 * w_fac,
           "hbm_bytes_per_launch": fa * 1024 * f_fac + wa * 1024 * w_fac,
           "note": "L2 fills from and write-backs to the data fabric: HBM plus MALL hits, so an upper "
                   "bound on the HBM bytes",
           "source_sha256": source_sha(os.path.join(CSRC, src)),
           "source_sha256_of": f"{src} with comments and blank space removed (the code the counters were taken on)",
           "command": command}
    with open(traffic_path(op, workload), "w") as f:
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


# ---------------------------------------------------- CPU oracle workers --
_MMAP = {}


def _mm(path):
    a = _MMAP.get(path)
    if a is None:
        import numpy as np
        a = np.load(path, mmap_mode="r")
        _MMAP[path] = a
    return a


def _worker_init():
    # one BLAS thread per worker process: the variables must be set before
    # numpy loads its BLAS (the workers are forked before the parent imports
    # numpy), and threadpool_limits then covers a BLAS already loaded
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401
    from threadpoolctl import threadpool_limits
    globals()["_LIMIT"] = threadpool_limits(limits=1)


def _task_indexer(job):
    """Oracle indexer + top-k of some query rows of one sequence: the keys the
    rows reach are decoded once (O.key_matrix), then each row is scored
    (O.indexer_scores) and selected (O.select_topk), as O.indexer_topk does
    for a whole sequence.  Returns the rows' indices and the task's time, its
    decode time and decoded key rows, and its per-row time."""
    import numpy as np
    from oracle import dsa_oracle as O
    t0 = time.perf_counter()
    n_dec = min(max(job["pos"]), job["kv_len"] - 1) + 1
    sc = None if job["scale"] is None else _mm(job["scale"])[:n_dec]
    kmat = O.key_matrix(_mm(job["keys"])[:n_dec], job["kd"], sc)
    t1 = time.perf_counter()
    res = np.full((len(job["pos"]), job["k"]), -1, dtype=np.int32)
    for i, p in enumerate(job["pos"]):
        n = min(p, job["kv_len"] - 1) + 1
        s = O.indexer_scores(O.decode_bf16(job["q"][i]), np.asarray(job["w"][i], np.float64), kmat[:n])
        res[i] = O.select_topk(s, job["k"])
    t2 = time.perf_counter()
    return job["tag"], res, t2 - t0, t1 - t0, n_dec, t2 - t1


def _task_attention(job):
    """Oracle sparse attention of some query rows over their gathered latent
    rows (slot j of row i is row i*k + j of the gathered block)."""
    from oracle import dsa_oracle as O
    t0 = time.perf_counter()
    kvg = _mm(job["kv"])[job["r0"]:job["r1"]]                      # [R, k, D]
    o, _ = O.sparse_attention(job["Q"], kvg, job["slot"], kvg.shape[1], job["sm"], job["d_v"])
    return job["tag"], o, time.perf_counter() - t0


def _worker_blas():
    from threadpoolctl import threadpool_info
    return [(p.get("internal_api"), p.get("num_threads")) for p in threadpool_info() if p.get("user_api") == "blas"]


def cpu_info():
    """What the oracle runs on: CPU model, visible cores, numpy and BLAS."""
    import numpy as np
    info = {"logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            key, _, val = line.partition(":")
            if key.strip() in ("Model name", "Socket(s)", "Core(s) per socket", "Thread(s) per core"):
                info[key.strip()] = val.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [f"{p.get('internal_api')} {p.get('version')} ({os.path.basename(p.get('filepath', ''))})"
                        for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:  # noqa: BLE001 - informational only
        pass
    return info


class OraclePool:
    """Worker processes for the CPU oracle, one BLAS thread each.  They are
    forked before this process touches the GPU, so they carry no device
    state.  Large inputs go to them as .npy files they memory-map."""

    def __init__(self, n):
        import multiprocessing as mp
        self.n = n
        self.pool = mp.get_context("fork").Pool(n, initializer=_worker_init)
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.dir = tempfile.mkdtemp(prefix="ix_oracle_", dir=base)
        self._k = 0

    def put(self, arr):
        import numpy as np
        self._k += 1
        path = os.path.join(self.dir, f"a{self._k}.npy")
        np.save(path, np.ascontiguousarray(arr))
        return path

    def run(self, fn, jobs):
        """(results in job order, wall seconds, summed task seconds)."""
        t0 = time.perf_counter()
        res = self.pool.map(fn, jobs, chunksize=1)
        return res, time.perf_counter() - t0, sum(r[2] for r in res)

    def close(self):
        self.pool.terminate()
        self.pool.join()
        shutil.rmtree(self.dir, ignore_errors=True)


def _chunks(seq, n):
    return [seq[i:i + n] for i in range(0, len(seq), n)]


def gathered_kv(torch, kv_b, idx_rows):
    """Host copy of the latent rows each query row attends over, [R, k, D]
    bf16 bits, and the slot map [R, 1, k] (-1 where idx is -1)."""
    import numpy as np
    g = kv_b[idx_rows.clamp(min=0).long()]                          # [R, k, D] on the device
    bits = g.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    k = idx_rows.shape[-1]
    slot = torch.where(idx_rows >= 0, torch.arange(k, device=idx_rows.device).view(1, k),
                       torch.full_like(idx_rows, -1))
    return bits, slot.view(-1, 1, k).cpu().numpy().astype(np.int32)


def cpu_baseline(w, inp, torch, rows, pool):
    """The oracle on the sampled query rows of every layer (indexer + top-k on
    the full layers, attention given the GPU's indices on all), over the
    worker pool; the sample's wall time is extrapolated to the whole step by
    the per-row cost model (indexer and top-k ~ candidates per row, attention
    ~ min(k, candidates))."""
    import numpy as np

    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    sm = 1.0 / math.sqrt(w.d_qk)
    ix_jobs, at_jobs = [], []
    f = -1
    rows_t = torch.tensor(rows, device=inp.idx_fs.device)
    for l in range(w.n_layers):
        if w.roles[l] == "F":
            f += 1
            e = inp.ix[l]
            kd = "bf16" if e["keys"].dtype == torch.bfloat16 else "fp8"
            kb = bits(e["keys"][0]) if kd == "bf16" else e["keys"][0].view(torch.uint8).cpu().numpy()
            kpath = pool.put(kb)
            spath = None if e["k_scale"] is None else pool.put(e["k_scale"][0].cpu().numpy())
            q, wt = bits(e["q"][0, rows_t]), e["w"][0, rows_t].cpu().numpy()
            # one job per worker, rows dealt round-robin from the longest so
            # the jobs carry similar work
            order = sorted(range(len(rows)), key=lambda i: -rows[i])
            for j in range(min(pool.n, len(rows))):
                grp = order[j::pool.n]
                ix_jobs.append(dict(tag=(f, grp), q=q[grp], w=wt[grp], keys=kpath, kd=kd, scale=spath,
                                    pos=[w.q_start + rows[i] for i in grp], kv_len=w.kv_len, k=w.k))
        a = inp.attn[l]
        kvg, slot = gathered_kv(torch, a["kv"][0], inp.idx_fs[f][0, rows_t])
        kvpath = pool.put(kvg)
        Q = bits(a["q"][0, rows_t])                                   # [R, Hq, D]
        for grp in _chunks(list(range(len(rows))), 8):
            r0, r1 = grp[0], grp[-1] + 1
            at_jobs.append(dict(tag=(l, r0, r1), Q=Q[r0:r1, None], kv=kvpath, r0=r0, r1=r1, slot=slot[r0:r1],
                                sm=sm, d_v=w.d_v))
    ix_res, ix_wall, ix_sum = pool.run(_task_indexer, ix_jobs)
    at_res, at_wall, at_sum = pool.run(_task_attention, at_jobs)
    n_f = w.roles.count("F")
    idx_oracle = [np.full((len(rows), w.k), -1, np.int32) for _ in range(n_f)]
    for (fi, grp), res, *_ in ix_res:
        idx_oracle[fi][grp] = res
    outs = [np.zeros((len(rows), w.q_heads, w.d_v)) for _ in range(w.n_layers)]
    for (l, r0, r1), o, _ in at_res:
        outs[l][r0:r1] = o[:, 0]
    # whole step in worker seconds: each full layer decodes every key row once
    # (at the sample's decode rate), each row costs its sample rate times its
    # candidates (indexer) or min(k, candidates) (attention); the rows are
    # independent, so the pool's wall time is that over its workers
    samp_pairs = sum(w.q_start + t + 1 for t in rows)
    samp_rows = sum(min(w.k, w.q_start + t + 1) for t in rows)
    dec_s = sum(r[3] for r in ix_res) / sum(r[4] for r in ix_res)        # seconds per decoded key row
    row_s = sum(r[5] for r in ix_res) / n_f
    full_worker_s = (n_f * w.batch * w.kv_len * dec_s + n_f * row_s * causal_pairs(w) / samp_pairs
                     + at_sum * gathered_rows(w) / samp_rows)
    return dict(t_ix=ix_wall, t_at=at_wall, t_sum=ix_sum + at_sum, full_s=full_worker_s / pool.n,
                full_worker_s=full_worker_s, idx=idx_oracle, O=outs, n_f=n_f, samp_rows=len(rows))


def sampled_parity(w, inp, rows, cb, torch):
    """GPU vs oracle on the sampled rows: index-set overlap per full layer
    (summed and worst row) and max-abs error of every layer's output given
    the GPU's indices."""
    import numpy as np

    ovl, worst = [], 1.0
    for f, ref in enumerate(cb["idx"]):
        got = inp.idx_fs[f][0, rows].cpu().numpy()
        inter = tot = 0
        for g, r in zip(got, ref):
            sr = set(r[r >= 0].tolist())
            i = len(set(g[g >= 0].tolist()) & sr)
            inter += i
            tot += len(sr)
            worst = min(worst, i / max(len(sr), 1))
        ovl.append(inter / max(tot, 1))
    err = max(float(np.abs(inp.attn[l]["out"][0, rows].float().cpu().numpy() - cb["O"][l]).max())
              for l in range(w.n_layers))
    return {"rows": len(rows), "idx_overlap_min": min(ovl), "idx_overlap_worst_row": worst,
            "attn_max_abs_err": err, "ok": min(ovl) >= 0.999 and err <= 2e-2}


def cpu_block(value, unit, pool, info, sample):
    info = dict(info, worker_blas_threads=pool.pool.apply(_worker_blas))
    return {"value": value, "unit": unit, "cores": pool.n, "kind": "oracle", "sample": sample,
            "workers": f"{pool.n} processes x 1 BLAS thread (capped at the {HOST_CPU_SHARE}-core CPU share "
                       f"of one GPU, or the cores this process may run on)", "host": info}


# ------------------------------------------------------------------ main --
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
                    help="rows checked against the oracle and timed on the CPU (0: 64, fewer for "
                         "rows of more than 512K candidates so the CPU leg stays near half a minute)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-full", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, copy a 1 GiB device buffer 4 times (HBM counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write a kernel's traffic summary from two rocprofv3 --pmc output dirs")
    ap.add_argument("--traffic-op", choices=sorted(TRAFFIC_OPS), default="attention")
    ap.add_argument("--traffic-command", default="", help="command recorded with --write-traffic")
    ap.add_argument("--fp8-queries", action="store_true",
                    help="--op indexer/argmax: e4m3fn queries with a per-(row, head) scale")
    ap.add_argument("--op", choices=["indexer", "argmax", "attention", "project", "topk"],
                    help="time one op of the workload's first layer alone (warmup + steps launches), for profiling; "
                         "topk: ix_topk_scores on 32 rows x 200,001 fp32 scores, whatever the workload")
    args = ap.parse_args(argv)
    if args.write_traffic:
        write_traffic(args.traffic_op, CONFIGS[args.config], *args.write_traffic, args.traffic_command)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the DSA group path runs on exactly one GPU; it has no multi-GPU "
                          "mode, so --gpus must be 1"}))
        return 2

    pool = None
    if not args.no_cpu_baseline and not args.op:
        # before anything touches the GPU: the workers are forked copies of
        # this process and must not inherit device state
        pool = OraclePool(min(HOST_CPU_SHARE, len(os.sched_getaffinity(0))))
    try:
        return run(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run(args, pool):
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
        return bench_decode(args, w, torch, synth, ix, pool)

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
    # the same score stream with a running maximum in place of the streaming
    # top-k: the difference is what the fused top-k costs
    am_pos = torch.empty((w.batch, w.n_q), dtype=torch.int32, device="cuda")
    am_ms = event_time(torch, lambda: ix.ix_indexer_argmax(e["q"], e["w"], e["keys"], am_pos, k_scale=e["k_scale"],
                                                           q_start=w.q_start, kv_len=w.kv_len), args.kernel_reps)
    a = inp.attn[1]
    at_ms = event_time(torch, lambda: ix.ix_sparse_attn(a["q"], a["kv"], idx0, a["out"], q_start=w.q_start,
                                                        kv_len=w.kv_len), args.kernel_reps)
    ix_flop = causal_pairs(w) * 2 * w.ix_heads * w.ix_dim
    ix_tflops = ix_flop / (ix_ms / 1e3) / 1e12
    g_rows = gathered_rows(w)
    at_bytes = g_rows * w.d_qk * 2 + w.batch * w.n_q * (w.q_heads * (w.d_qk + w.d_v) * 2 + w.k * 4)
    at_gbps = at_bytes / (at_ms / 1e3) / 1e9
    at_flop = g_rows * w.q_heads * 2 * (w.d_qk + w.d_v)
    ix_alg_bytes = w.batch * (w.n_q * (w.ix_heads * w.ix_dim * 2 + w.ix_heads * 4 + w.k * 4)
                              + w.kv_len * (w.ix_dim * (1 if w.key_dtype == "fp8" else 2)
                                            + (4 if w.key_dtype == "fp8" else 0)))

    # standalone row top-k over materialised fp32 rows at the decode shape
    # (32 rows of 200,001 scores): HBM fraction on one read of the rows.  A
    # call is ~20 us of GPU work, so it is timed over 100 back-to-back calls
    # (over a handful, the host's launch of each call shows in the figure)
    g = torch.Generator(device="cuda").manual_seed(0)
    dk = synth.DECODE_B32
    tk_scores = torch.randn((dk.batch, 1, dk.kv_len), generator=g, device="cuda")
    tk_idx = torch.empty((dk.batch, 1, dk.k), dtype=torch.int32, device="cuda")
    tk_ms = event_time(torch, lambda: ix.ix_topk_scores(tk_scores, tk_idx, q_start=dk.q_start, kv_len=dk.kv_len),
                       max(args.kernel_reps, 100))
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

    log("indexer projection")
    project = project_leg(w, torch, synth, ix, args.kernel_reps)

    log("fp8-query indexer")
    fp8q = fp8_query_leg(w, torch, synth, ix, inp, run_group, fs_mask, args, ix_ms, ix_flop)

    allf_ms = None
    if not args.no_all_full:
        log("all-full baseline")
        allf_mask = (1 << w.n_layers) - 1
        allf_ms = event_time(torch, lambda: run_group(allf_mask, inp.idx_ff), 1)
        # all-F baseline re-ran the F layers' slots; restore the F+3S indices
        run_group(fs_mask, inp.idx_fs)
        torch.cuda.synchronize()

    ix_tr, at_tr = load_traffic("indexer", w.name), load_traffic("attention", w.name)
    ix_traffic = None if ix_tr is None else ix_tr["hbm_bytes_per_launch"]
    at_traffic = None if at_tr is None else at_tr["hbm_bytes_per_launch"]

    n_sample = args.sample_rows
    if n_sample <= 0:   # the oracle costs about 2 s per row at 1M candidates
        n_sample = 64 if w.kv_len <= 512 * 1024 else 16
    rows = synth.sample_rows(w, n_sample)
    result_cpu, parity = None, None
    if pool is not None:
        log(f"CPU oracle on {len(rows)} sampled rows, {pool.n} worker processes")
        cb = cpu_baseline(w, inp, torch, rows, pool)
        n_tokens = w.batch * w.n_q
        result_cpu = cpu_block(
            n_tokens / (cb["full_s"] / n_groups), "tokens/s per group", pool, cpu_info(),
            f"{len(rows)} query rows of {w.n_q} (first and last rows, rows with k-1, k, k+1 candidates, "
            f"the rest seeded-uniform) through all {w.n_layers} layers (indexer + top-k on {cb['n_f']} full "
            f"layers, attention given the GPU's indices): {cb['t_ix'] + cb['t_at']:.1f} s wall on the pool "
            f"({cb['t_sum']:.1f} s of worker time); extrapolated to the whole step ({cb['full_worker_s']:.0f} "
            f"worker-s, spread over the {pool.n} workers) by one key decode per full layer and, per row, its "
            f"candidates (indexer) or min(k, candidates) (attention)")
        parity = sampled_parity(w, inp, rows, cb, torch)

    topk_ms = ix_ms - am_ms
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
        "roofline": {"bound": "mfma", "achieved": ix_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ix_tflops / PEAK_BF16_TFLOPS, "traffic": ix_traffic,
                     "kernel": "fused_indexer_topk_kernel (+ its key staging, 0.01% of the call): 2*H*d FLOP per "
                               "causal (row, key) pair on bf16 MFMA (fp8 keys widened exactly); traffic = HBM "
                               "bytes per launch from calibrated FETCH_SIZE + WRITE_SIZE",
                     "algorithmic_bytes": ix_alg_bytes},
        "indexer": {"ms": ix_ms, "tflops": ix_tflops, "frac_bf16_peak": ix_tflops / PEAK_BF16_TFLOPS,
                    "frac_fp8_peak": ix_tflops / PEAK_FP8_TFLOPS, "flop": ix_flop,
                    "traffic_over_algorithmic": None if ix_traffic is None else ix_traffic / ix_alg_bytes,
                    "note": "fused score + streaming top-k, incl. staging the keys as bf16 (fp8 widened exactly)"},
        "fused_topk": {"ms": topk_ms, "rows_per_s": w.batch * w.n_q / (topk_ms / 1e3) if topk_ms > 0 else None,
                       "candidates_per_s": causal_pairs(w) / (topk_ms / 1e3) if topk_ms > 0 else None,
                       "share_of_indexer": topk_ms / ix_ms, "argmax_ms": am_ms,
                       "note": "indexer with streaming top-k minus the same score stream with a running maximum "
                               "(ix_indexer_argmax); its HBM bytes are the candidate-buffer traffic in "
                               "roofline.traffic"},
        "attention": {"ms_per_layer": at_ms, "tokens_per_s": w.batch * w.n_q / (at_ms / 1e3),
                      "gathered_GBps_cache_served": at_gbps, "gathered_bytes_per_launch": at_bytes,
                      "fabric_bytes_per_launch": at_traffic,
                      "fabric_GBps": None if at_traffic is None else at_traffic / (at_ms / 1e3) / 1e9,
                      "hbm_frac_upper_bound": None if at_traffic is None
                      else at_traffic / (at_ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
                      "tflops": at_flop / (at_ms / 1e3) / 1e12,
                      "note": "gathered bytes are served largely from L2 and the MALL (neighbouring rows select "
                              "overlapping latent rows), so their rate is not an HBM rate; fabric bytes "
                              "(calibrated FETCH_SIZE + WRITE_SIZE) bound the HBM bytes from above"},
        "topk_standalone": {"workload": "32 rows x 200,001 fp32 scores, k=2048", "us": tk_ms * 1e3,
                            "rows_per_s": dk.batch / (tk_ms / 1e3),
                            "frac_hbm_peak": tk_bytes / (tk_ms / 1e3) / 1e9 / PEAK_HBM_GBPS},
        "index_overlap": overlap,
        "project": project,
        "fp8_queries": fp8q,
        "group": {"ms_fsss": ms_step / n_groups, "ms_all_full": None if allf_ms is None else allf_ms / n_groups,
                  "speedup_vs_all_full": None if allf_ms is None else allf_ms / ms_step},
        "cpu_baseline": result_cpu,
        "parity": parity,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        copy_calibration(torch)
    return 0


def copy_calibration(torch):
    src = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()


def fp8_query_leg(w, torch, synth, ix, inp, run_group, fs_mask, args, ix_ms, ix_flop):
    """The declared fp8-query mode: every full layer's bf16 queries quantised
    by ix_quantize_queries to e4m3fn codes with a per-(row, head) scale
    (amax / 448, the fp8 key recipe).  Times the quantiser, the indexer call
    and the whole group step in that mode, and counts how many of the
    bf16-query run's positions the fp8-query run selects too.  The headline
    value stays the bf16-query step."""
    saved = list(inp.ix)
    for l, e in enumerate(saved):
        if e is not None:
            codes, qs = ix.ix_quantize_queries(e["q"])
            inp.ix[l] = dict(e, q=codes, q_scale=qs)
    idx8 = torch.empty_like(inp.idx_fs)
    try:
        e = inp.ix[0]
        q16 = saved[0]["q"]
        qz_ms = event_time(torch, lambda: ix.ix_quantize_queries(q16, e["q"], e["q_scale"]), args.kernel_reps)
        ms = event_time(torch, lambda: ix.ix_indexer_topk(e["q"], e["w"], e["keys"], idx8[0], k_scale=e["k_scale"],
                                                          q_start=w.q_start, kv_len=w.kv_len,
                                                          q_scale=e["q_scale"]), args.kernel_reps)
        step_ms = event_time(torch, lambda: ix.ix_group_forward(inp.ix, inp.attn, fs_mask, idx8, q_start=w.q_start,
                                                                kv_len=w.kv_len), max(1, args.steps))
    finally:
        inp.ix[:] = saved
        run_group(fs_mask, inp.idx_fs)        # the attention outputs of the bf16-query step again
        torch.cuda.synchronize()
    same = ix.ix_index_overlap(inp.idx_fs[0], idx8[0]).float()
    valid = (inp.idx_fs[0] >= 0).sum(dim=-1).clamp(min=1).float()
    frac = same / valid
    del idx8
    n_groups = w.n_layers // 4
    tflops = ix_flop / (ms / 1e3) / 1e12
    fp8_form = w.key_dtype == "fp8" and w.ix_dim in (64, 128)
    qz_bytes = q16.numel() * 3 + q16[..., 0].numel() * 4      # bf16 read, codes + scales written
    return {"quantize_ms": qz_ms, "quantize_frac_hbm_peak": qz_bytes / (qz_ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
            "indexer_ms": ms, "tflops": tflops, "frac_fp8_peak": tflops / PEAK_FP8_TFLOPS,
            "indexer_speedup_vs_bf16_queries": ix_ms / ms, "ms_per_group": step_ms / n_groups,
            "tokens_per_s_per_group": w.batch * w.n_q / (step_ms / n_groups / 1e3),
            "overlap_with_bf16_query_indices": {"mean": float(frac.mean()), "min_row": float(frac.min())},
            "note": ("fp8 MFMA on the cached e4m3fn keys read in place" if fp8_form
                     else "codes widened to bf16 (no fp8 MFMA form for these keys)")
            + "; the first full layer's queries quantised per (row, head); a mode the caller declares, so not "
              "the headline value"}


def project_leg(w, torch, synth, ix, reps):
    """The indexer projection (q_I and head weights from hidden states) at the
    workload's rows: time, TFLOP/s against the bf16 MFMA peak."""
    x, wp = synth.projection_inputs(w, "cuda")
    rows, d_in = x.shape
    q = torch.empty((rows, w.ix_heads, w.ix_dim), dtype=torch.bfloat16, device="cuda")
    wo = torch.empty((rows, w.ix_heads), dtype=torch.float32, device="cuda")
    fn = lambda: ix.ix_indexer_project(x, wp, q, wo, heads=w.ix_heads, dim=w.ix_dim)
    fn()
    ms = event_time(torch, fn, reps)
    flop = 2.0 * rows * wp.shape[0] * d_in
    tflops = flop / (ms / 1e3) / 1e12
    return {"shape": f"{rows} x {d_in} -> {w.ix_heads} x {w.ix_dim} + {w.ix_heads}", "ms": ms, "us": ms * 1e3,
            "tflops": tflops, "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
            "weight_GBps": wp.numel() * 2 / (ms / 1e3) / 1e9,
            "note": "ix_indexer_project: one GEMM on bf16 MFMA, q_I rounded to bf16, head weights fp32"}


def bench_op(args, w, torch, synth, ix):
    """One op of the first layer, launched warmup + steps times: the indexer
    (+ fused top-k), the same score stream with a running maximum
    (ix_indexer_argmax), the sparse attention over the indexer's positions,
    the indexer projection, or (topk) the standalone row top-k at the decode
    shape."""
    dev = "cuda"
    if args.op == "project":
        x, wp = synth.projection_inputs(w, dev)
        pq = torch.empty((x.shape[0], w.ix_heads, w.ix_dim), dtype=torch.bfloat16, device=dev)
        pw = torch.empty((x.shape[0], w.ix_heads), dtype=torch.float32, device=dev)
        fn = lambda: ix.ix_indexer_project(x, wp, pq, pw, heads=w.ix_heads, dim=w.ix_dim)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ms = event_time(torch, fn, args.steps) if args.steps > 0 else None
        print(json.dumps({"op": args.op, "workload": w.name, "launches": args.warmup + args.steps + 1,
                          "ms_per_launch": ms}), flush=True)
        return 0
    if args.op == "topk":
        dk = synth.DECODE_B32
        g = torch.Generator(device=dev).manual_seed(0)
        scores = torch.randn((dk.batch, 1, dk.kv_len), generator=g, device=dev)
        idx = torch.empty((dk.batch, 1, dk.k), dtype=torch.int32, device=dev)
        fn = lambda: ix.ix_topk_scores(scores, idx, q_start=dk.q_start, kv_len=dk.kv_len)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ms = event_time(torch, fn, args.steps) if args.steps > 0 else None
        print(json.dumps({"op": args.op, "workload": "32 rows x 200,001 fp32 scores, k=2048",
                          "launches": args.warmup + args.steps + 1, "ms_per_launch": ms}), flush=True)
        if args.copy_calibration:
            copy_calibration(torch)
        return 0
    qs = None
    if args.fp8_queries:
        q, qs, wt = synth.indexer_queries_fp8(w, dev, 0)
    else:
        q, wt = synth.indexer_queries(w, dev, 0)
    keys, scale = synth.indexer_keys(w, dev, 0)
    idx = torch.empty((w.batch, w.n_q, w.k), dtype=torch.int32, device=dev)
    run_ix = lambda: ix.ix_indexer_topk(q, wt, keys, idx, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len,
                                        q_scale=qs)
    fn = run_ix
    if args.op == "argmax":
        pos = torch.empty((w.batch, w.n_q), dtype=torch.int32, device=dev)
        fn = lambda: ix.ix_indexer_argmax(q, wt, keys, pos, k_scale=scale, q_start=w.q_start, kv_len=w.kv_len,
                                          q_scale=qs)
    if args.op == "attention":
        run_ix()
        del q, qs, wt, keys, scale
        aq = synth.attn_queries(w, dev, 0)
        kv = synth.latent_kv(w, dev, 0)
        out = torch.empty((w.batch, w.n_q, w.q_heads, w.d_v), dtype=torch.bfloat16, device=dev)
        fn = lambda: ix.ix_sparse_attn(aq, kv, idx, out, q_start=w.q_start, kv_len=w.kv_len)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    ms = event_time(torch, fn, args.steps) if args.steps > 0 else None
    print(json.dumps({"op": args.op, "workload": w.name, "launches": args.warmup + args.steps + 1,
                      "fp8_queries": bool(args.fp8_queries), "ms_per_launch": ms}), flush=True)
    if args.copy_calibration:
        copy_calibration(torch)
    return 0


def decode_oracle_leg(w, torch, keys, scale, kvs, step_inputs, last, j, log, pool):
    """The CPU oracle on every sequence of decode step j (indexer over the
    whole cache, then the four layers' attention over the GPU's positions)
    over the worker pool; parity of those sequences."""
    import numpy as np

    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    q_start, kv_len = w.q_start + j, w.kv_len + j
    ixl, att = step_inputs
    ixe = ixl[0]                                   # the full layer's indexer inputs
    gpu_idx = last["idx"]                          # [B, 1, k]
    log(f"CPU oracle on {w.batch} sequences of decode step {j}, {pool.n} worker processes")
    ix_jobs = []
    for b in range(w.batch):
        kpath = pool.put(keys[b, :kv_len].contiguous().cpu().numpy())
        spath = pool.put(scale[b, :kv_len].cpu().numpy())
        ix_jobs.append(dict(tag=b, q=bits(ixe["q"][b]), w=ixe["w"][b].cpu().numpy(), keys=kpath, kd="fp8",
                            scale=spath, pos=[q_start], kv_len=kv_len, k=w.k))
    at_jobs = []
    for l in range(4):
        g = torch.stack([kvs[l][b][gpu_idx[b, 0].clamp(min=0).long()] for b in range(w.batch)])   # [B, k, D]
        kvpath = pool.put(bits(g))
        slot = torch.where(gpu_idx >= 0, torch.arange(w.k, device=keys.device).view(1, 1, -1),
                           torch.full_like(gpu_idx, -1)).cpu().numpy().astype(np.int32)
        Q = bits(att[l]["q"])                                             # [B, 1, Hq, D]
        for grp in _chunks(list(range(w.batch)), 4):
            r0, r1 = grp[0], grp[-1] + 1
            at_jobs.append(dict(tag=(l, r0, r1), Q=Q[r0:r1], kv=kvpath, r0=r0, r1=r1, slot=slot[r0:r1],
                                sm=1.0 / math.sqrt(w.d_qk), d_v=w.d_v))
    ix_res, ix_wall, ix_sum = pool.run(_task_indexer, ix_jobs)
    at_res, at_wall, at_sum = pool.run(_task_attention, at_jobs)
    ref_idx = np.stack([r[1][0] for r in ix_res])                     # [B, k]
    got = gpu_idx[:, 0].cpu().numpy()
    inter = tot = 0
    worst = 1.0
    for g, r in zip(got, ref_idx):
        sr = set(r[r >= 0].tolist())
        i = len(set(g[g >= 0].tolist()) & sr)
        inter += i
        tot += len(sr)
        worst = min(worst, i / max(len(sr), 1))
    ovl = inter / max(tot, 1)
    err = 0.0
    for (l, r0, r1), o, _ in at_res:
        err = max(err, float(np.abs(last["outs"][l][r0:r1].float().cpu().numpy() - o).max()))
    step_s = ix_wall + at_wall
    cpu = cpu_block(w.batch / step_s, "tokens/s", pool, cpu_info(),
                    f"all {w.batch} sequences of decode step {j} (indexer + top-k over {kv_len:,} keys, 4 layers "
                    f"of attention given the GPU's indices): {step_s:.1f} s wall on the pool "
                    f"({ix_sum + at_sum:.1f} s of worker time)")
    parity = {"sequences": w.batch, "idx_overlap": ovl, "idx_overlap_worst_row": worst,
              "attn_max_abs_err": err, "ok": ovl >= 0.999 and err <= 2e-2}
    return cpu, parity


def bench_decode(args, w, torch, synth, ix, pool):
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
    # fp8 keys, then the one-pass merge), about 60% of the step
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
    at_ms = event_time(torch, lambda: ix.ix_sparse_attn(steps[j_last][1][1]["q"], kvs[1], ix_idx,
                                                        steps[j_last][1][1]["out"], q_start=w.q_start + j_last,
                                                        kv_len=w.kv_len + j_last), 20)
    at_bytes = w.batch * w.k * w.d_qk * 2
    attention = {"us_per_layer": at_ms * 1e3, "gathered_GBps": at_bytes / (at_ms / 1e3) / 1e9,
                 "gathered_bytes": at_bytes}

    project = project_leg(w, torch, synth, ix, 50)

    result_cpu, parity = None, None
    if pool is not None:
        result_cpu, parity = decode_oracle_leg(w, torch, keys, scale, kvs, steps[j_last], last, j_last, log, pool)
    out = {"metric": "decode tokens/s (B=32, 200K context, one F,S,S,S group per step)",
           "value": w.batch / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, on device)",
           "config": {"workload": w.name, "batch": w.batch, "context": w.kv_len, "k": w.k},
           "step": "quantize+append the new token's indexer key into the fp8 cache, then the F,S,S,S group",
           "roofline": roofline, "cpu_baseline": result_cpu, "parity": parity,
           "append_keys_us": app_ms * 1e3, "attention": attention,
           "group": {"ms_fsss": ms, "ms_all_full": allf, "speedup_vs_all_full": allf / ms},
           "varlen": varlen, "mtp_draft": mtp, "project": project,
           "indexer_key_GBps_lower_bound": key_bytes / (ms / 1e3) / 1e9}
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
