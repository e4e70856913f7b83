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
import re
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


# Per-kernel limits checked on the compiler's resource report: no kernel may
# use scratch (private) memory, and none may need more than 256 registers
# per lane (VGPRs + AGPRs). Above 256 the compiler parks values in the
# accumulation registers and spills scalar registers into vector lanes; one
# such variant returned wrong eigenvectors on the GPU with its cause not
# found, so the build provides none.
MAX_REGS_PER_LANE = 256
RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def parse_resource_usage(text: str) -> dict:
    """Kernel name -> {field: int} from the compiler's resource remarks."""
    out: dict = {}
    cur = None
    for line in text.splitlines():
        if RESOURCE_REMARK[2:] not in line:
            continue
        # "<file>:<line>:<col>: remark: <body> [-R...]" or
        # "remark: <file>:<line>:<col>: <body> [-R...]"
        m = re.search(r":\d+:\d+:\s+(?:remark:\s+)?(.*?)\s*\[-R", line)
        if not m:
            continue
        body = m.group(1)
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in body:
            key, val = body.rsplit(":", 1)
            val = val.strip()
            if val.lstrip("-").isdigit():
                out[cur][key.strip()] = int(val)
    return out


# Producer-consumer shapes whose register budget is fixed by the workgroup
# (12 or 11 wavefronts per CU, three per SIMD: 168 registers per lane) and
# which keep a few bytes per lane in scratch memory (measured by this
# report): a value held across the pass loop (double, order 64, and float,
# order 128: 12 bytes), never touched by the chase or the rotation of Q;
# and the double order-256 and order-512 shapes, whose 36- and 52-byte
# private segments no instruction accesses (their device assembly holds no
# scratch load or store). Any other kernel with scratch fails the build.
SCRATCH_ALLOWED = {
    "_ZN5steqr15steqr_pc_kernelIdLi64ELi11ELi4ELb0ELb1ELi1EEEvNS_10KernelArgsE": 12,
    "_ZN5steqr15steqr_pc_kernelIdLi64ELi11ELi4ELb1ELb1ELi1EEEvNS_10KernelArgsE": 12,
    "_ZN5steqr15steqr_pc_kernelIfLi128ELi10ELi8ELb0ELb1ELi1EEEvNS_10KernelArgsE": 12,
    "_ZN5steqr15steqr_pc_kernelIfLi128ELi10ELi8ELb1ELb1ELi1EEEvNS_10KernelArgsE": 12,
    "_ZN5steqr15steqr_pc_kernelIdLi256ELi8ELi64ELb0ELb1ELi4EEEvNS_10KernelArgsE": 36,
    "_ZN5steqr15steqr_pc_kernelIdLi256ELi8ELi64ELb1ELb1ELi4EEEvNS_10KernelArgsE": 36,
    "_ZN5steqr15steqr_pc_kernelIdLi512ELi8ELi64ELb0ELb1ELi16EEEvNS_10KernelArgsE": 52,
    "_ZN5steqr15steqr_pc_kernelIdLi512ELi8ELi64ELb1ELb1ELi16EEEvNS_10KernelArgsE": 52,
}


def check_resources(usage: dict, src: str) -> None:
    bad = []
    for name, u in usage.items():
        regs = u.get("VGPRs", 0) + u.get("AGPRs", 0)
        scratch = u.get("ScratchSize [bytes/lane]", 0)
        if scratch > SCRATCH_ALLOWED.get(name, 0) or regs > MAX_REGS_PER_LANE:
            bad.append("%s: %d VGPRs + %d AGPRs, scratch %d bytes/lane"
                       % (name, u.get("VGPRs", 0), u.get("AGPRs", 0), scratch))
    if bad:
        raise RuntimeError("kernels over the register / scratch limits in %s:\n  %s"
                           % (os.path.basename(src), "\n  ".join(bad)))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, RESOURCE_REMARK, "-c", src, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "not a recognized feature for this target" not in l
                    and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    usage = parse_resource_usage(r.stderr)
    with open(obj + ".resources.txt", "w") as f:
        for name, u in sorted(usage.items()):
            f.write("%s %s\n" % (name, " ".join("%s=%d" % (k.split(" ")[0], v)
                                                for k, v in u.items())))
    check_resources(usage, src)
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
