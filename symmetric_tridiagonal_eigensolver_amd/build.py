"""Build the HIP library libsteqr.so for gfx950, in-tree.

Each csrc/*.hip translation unit is compiled to an object in parallel
(hipcc, --offload-arch=gfx950) and the objects are linked into
symmetric_tridiagonal_eigensolver_amd/libsteqr.so. Run as a module:
    python -m symmetric_tridiagonal_eigensolver_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsteqr.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from emitting packed FP32 VALU ops.
# Division and square root stay IEEE correctly rounded (the block scaling
# factors must equal the ones of the CPU reference bit for bit).
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math", "-ffp-contract=fast",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if verbose:
        print("  compiled %s (%.1fs)" % (os.path.basename(src), time.time() - t), flush=True)
    return obj


def build(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libsteqr.so; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under %s" % CSRC)
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    t0 = time.time()
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s in %.1fs" % (LIB, time.time() - t0), flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
