"""Build libcq.so (the C-ABI CQ library) in-tree for gfx950 with hipcc.

Usage:  python hadamard_rotated_codebook_amd/build.py  [--jobs N]

Always recompiles every source.  Packed-fp32 instructions are disabled for all
device code (-target-feature -packed-fp32-ops).
"""
import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcq.so")
SOURCES = ["api.hip", "rotate.hip", "matvec.hip", "matvec_mma.hip", "multi_matvec.hip", "w2a8.hip", "gather.hip", "gemm.hip", "quantize.hip", "noalloc.hip", "kv.hip", "probe.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Keep single-lane atomics as written: the wave-combining rewrite waits for
    # the atomic's return at once, which drains the matvec's load pipeline.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file flags.  The small-matrix kernel takes its activation arguments as
# leading scalars and has the dispatcher preload them into SGPRs.
EXTRA = {"multi_matvec.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=6"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return obj


def build(jobs=None, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
