"""Builds libix.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m long_context_sparse_ix_amd.build [--jobs N]

Every source compiles to its own object in parallel, then one shared library
is linked next to this file.  Packed-FP32 instruction selection is switched
off for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libix.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMAs accumulate in VGPRs; the default AGPR form made the attention
          # kernel copy its 128-register output accumulator between the two
          # register files on every 16-slot step
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
          f"-I{INCLUDE}", f"-I{CSRC}"]


# Sources whose kernels keep MFMA accumulators in AGPRs (the compiler's
# default form): the projection GEMM holds a 256-register accumulator per
# wave, which only the AGPR file can take next to its VGPRs.
AGPR_FORM = {"indexer_project.hip"}


def _flags(src: str) -> list:
    if os.path.basename(src) not in AGPR_FORM:
        return CFLAGS
    i = CFLAGS.index("-amdgpu-mfma-vgpr-form=1")
    return CFLAGS[:i - 1] + CFLAGS[i + 1:]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *_flags(src), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    print(build(args.jobs))


if __name__ == "__main__":
    sys.exit(main())
