"""Benchmark: batched symmetric tridiagonal eigensolver on one MI355X.

Default workload: float32, n = 16, eigenvectors (jobz=V), batch 32,768
matrices with d, e iid N(0,1) (seeded). One step = one launch of
steqr_batched over the whole batch, inputs already resident in HBM.

Prints ONE JSON line: matrices/s, microseconds per matrix, the roofline of
the kernel (VALU-bound: algorithmic flops per launch from the CPU oracle's
rotation counts, over the kernel's mean duration measured with HIP events
on the launch stream, against the published FP32/FP64 vector peak), and
the CPU oracle timed on the host cores over the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6}  # MI355X published vector peaks
HBM_PEAK_GBS = 8000.0
# non-packed vector rate: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2.4 GHz
PEAK_NONPACKED_TFLOPS = 78.6


def flops_per_matrix(stats: np.ndarray, n: int, jobz: bool) -> np.ndarray:
    """Algorithmic flops of one solve from the oracle's counts.

    stats[:, 0] implicit sweeps S, [:, 1] sweep rotations R, [:, 2] analytic
    2x2 solves J. Per rotation: ~40 flops for the Givens generation and the
    similarity update of the band, plus 6n for the column-pair update of Q
    (jobz=V). Per sweep: ~10 flops for the shift. Per 2x2 solve: ~25 flops
    plus 6n for Q.
    """
    S, R, J = (stats[:, k].astype(np.float64) for k in range(3))
    q = 6.0 * n if jobz else 0.0
    return R * (40.0 + q) + S * 10.0 + J * (25.0 + q)


def bytes_per_matrix(n: int, itemsize: int, jobz: bool, back_transform: bool = False) -> int:
    """Algorithmic HBM bytes: read d (n) and e (n-1), write lambda (n) and
    Q (n^2) for jobz=V; with back-transformation Q is also read (n^2)."""
    q = (n * n if jobz else 0) * (2 if back_transform else 1)
    return ((2 * n - 1) + n + q) * itemsize


# Sources each kernel family is compiled from (its hash guards committed
# counter records against kernel changes).
KERNEL_SOURCES = {
    "chunk": ["steqr_device.hpp", "syev_reduce.hpp", "steqr_chunk.hpp"],
    "chunkl": ["steqr_device.hpp", "syev_reduce.hpp", "steqr_chunk.hpp", "steqr_chunkl.hpp"],
    "wave": ["steqr_device.hpp", "syev_reduce.hpp", "steqr_chunk.hpp", "steqr_wave.hpp"],
    "pc": ["steqr_device.hpp", "syev_reduce.hpp", "steqr_chunk.hpp", "steqr_chunkl.hpp",
           "steqr_pc.hpp"],
    "bisect": ["steqr_device.hpp", "syev_reduce.hpp", "steqr_chunk.hpp", "steqr_bisect.hpp"],
}


def strip_comments(src: str) -> str:
    """C++ source without its comments and blank space (so that a record
    taken on some code stays valid when only the comments change)."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif src[i] == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


# statements of the profiling build's phase timers: they expand to nothing
# in the library (the compiled kernels are those of the source without them)
PHASE_TIMER_STMT = re.compile(r'(#include "steqr_phase\.hpp"|STEQR_PHASE_[A-Z]+(\([^()]*\))?;) ?')


def kernel_source_hash(family: str = "chunk") -> str:
    """Hash of the code (comments and phase-timer statements stripped) of a
    kernel family's sources."""
    h = hashlib.sha256()
    cs = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        src = strip_comments(open(os.path.join(cs, f)).read())
        h.update(PHASE_TIMER_STMT.sub("", src).encode())
    return h.hexdigest()[:16]


def kernel_family(plan: dict, jobz: bool, method: int = 0) -> str:
    """Kernel family a launch plan runs: bisection; producer and consumer
    wavefronts (band 3), or their producer alone (values only: at order 64
    with fewer than 64 lanes per problem, and above order 64); one problem
    per wavefront (64 lanes at order 64); the chunked kernel with the band
    in LDS or in registers."""
    if method:
        return "bisect"
    if plan["band_storage"] == 3 or (not jobz and plan["padded_n"] >= 64
                                     and (plan["lanes_per_problem"] < 64
                                          or plan["padded_n"] > 64)):
        return "pc"
    if plan["lanes_per_problem"] == 64:
        return "wave"
    return "chunkl" if plan["band_storage"] == 2 else "chunk"


def kernel_label(plan: dict, jobz: bool, dtype: str, family: str, scheme: int = 0) -> str:
    """Name of the kernel instantiation a launch plan runs (", PG" for the
    Parlett-Gray form of the step)."""
    return "steqr_%s_kernel<%s, N=%d, P=%d, %s%s>" % (
        family, "float" if dtype == "f32" else "double", plan["padded_n"],
        plan["lanes_per_problem"], "V" if jobz else "N", ", PG" if scheme else "")


def record_suffix(bt: bool, scheme: int, method: int) -> str:
    """Counter-record name suffix of a launch option set: back-transformation,
    the PG step or bisection (the default solve has none)."""
    return "_bt" if bt else ("_pg" if scheme else ("_bisect" if method else ""))


def counters_from_profiles(wname: str, jobz: bool, family: str, kernel: str, suffix: str = ""):
    """Per-launch counter record (HBM bytes, executed VALU instructions and
    FLOPs, replicated-batch instructions) committed under profiles/, or None
    when absent, taken on another kernel instantiation or on other kernel
    sources."""
    p = os.path.join(ROOT, "profiles", "counters_%s_%s%s.json" % (wname, "V" if jobz else "N",
                                                                   suffix))
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    if t.get("kernel_source_hash") != kernel_source_hash(family) or t.get("kernel") != kernel:
        return None
    return t


def bisect_flops_per_matrix(counts: np.ndarray, n: int) -> np.ndarray:
    """Algorithmic flops of the values-only bisection: 4n per Sturm count
    (d_i - x, the reciprocal of the pivot and the multiply-add, per
    position), from the oracle's count of Sturm counts per matrix."""
    return counts.astype(np.float64) * 4.0 * n


def cpu_baseline(d: np.ndarray, e: np.ndarray, jobz: bool, wname: str, scheme: int = 0,
                 Z: np.ndarray = None, method: int = 0):
    """The CPU oracle (as is) on the host cores over the same workload.
    method 1: the oracle's bisection; stats is then its Sturm counts."""
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    oracle.steqr(d[:64], e[:64], jobz)  # load / warm
    times = []
    stats = None
    # the full batch (its rotation counts give the algorithmic flops), run
    # again until about a second of wall time (some 10-30 s of CPU work on
    # the host's cores) and at least three runs have passed, unless one run
    # alone takes 10 s; the median run
    total = 0.0
    while True:
        t = time.perf_counter()
        if method == 1:
            _, _, stats = oracle.stebz(d, e, threads=cores, counts=True)
        else:
            _, _, _, stats = oracle.steqr(d, e, jobz, threads=cores, scheme=scheme, Z=Z)
        times.append(time.perf_counter() - t)
        total += times[-1]
        if times[0] >= 10.0 or (len(times) >= 3 and total >= 1.0) or len(times) >= 500:
            break
    tmed = statistics.median(times)
    nb = d.shape[0]
    # one-thread figure on a prefix of the batch bounded to about 10 s
    per1 = tmed * cores / nb
    m1 = int(min(nb, max(4, 10.0 / max(per1, 1e-9))))
    t = time.perf_counter()
    if method == 1:
        oracle.stebz(d[:m1], e[:m1], threads=1)
    else:
        oracle.steqr(d[:m1], e[:m1], jobz, threads=1, scheme=scheme,
                     Z=None if Z is None else Z[:m1])
    t1 = time.perf_counter() - t
    return {
        "value": nb / tmed, "unit": "matrices/s", "cores": cores, "kind": "oracle",
        "us_per_matrix": tmed / nb * 1e6,
        "sample": "full %s batch (%d matrices), median of %d run%s on %d threads"
                  % (wname, nb, len(times), "s" if len(times) > 1 else "", cores),
        "one_thread_us_per_matrix": t1 / m1 * 1e6,
        "one_thread_sample": "first %d matrices, one run on 1 thread" % m1,
    }, stats


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="steqr", choices=["steqr", "syev"],
                    help="steqr: tridiagonal solve (default); syev: the fused dense "
                         "eigensolver on a DENSE workload (s_*)")
    ap.add_argument("--workload", default=None,
                    choices=list(W.WORKLOADS) + list(W.DENSE_WORKLOADS))
    ap.add_argument("--jobz", default="V", choices=["V", "N"])
    ap.add_argument("--batch", type=int, default=0,
                    help="matrices per launch (0 = the workload's own batch; another batch "
                         "runs the default launch for that batch, without counter records)")
    ap.add_argument("--lanes", type=int, default=0, help="lanes per problem (0 = default)")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup (0 = default)")
    ap.add_argument("--band", type=int, default=0,
                    help="band storage: 0 default, 1 registers, 2 LDS")
    ap.add_argument("--scheme", default="exp", choices=["exp", "pg"],
                    help="form of the chase step: EXP (default) or PG (Parlett-Gray)")
    ap.add_argument("--method", default="qr", choices=["qr", "bisect"],
                    help="eigenvalue method: QR iteration (default) or values-only "
                         "bisection (needs --jobz N)")
    ap.add_argument("--back-transform", action="store_true",
                    help="Q holds a basis on entry (seeded random orthogonal) that the "
                         "rotations right-multiply in place; needs --jobz V")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-saturation", action="store_true",
                    help="skip the saturation check (the same kernel at twice the batch)")
    ap.add_argument("--no-named", action="store_true",
                    help="skip the secondary timing at the configuration's named lanes")
    ap.add_argument("--replicate", action="store_true",
                    help="lockstep-ideal batch: every chunk of a wavefront holds the same "
                         "matrix (each item repeated 64/P times); for divergence counters")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of solving, run a plain device-to-device copy of MIB MiB "
                         "per step (reference kernel for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (--gpus %d requested); "
              "the batch is independent per matrix and would shard by contiguous slices, "
              "but no multi-GPU path is provided." % args.gpus, file=sys.stderr)
        return 2

    import torch
    import symmetric_tridiagonal_eigensolver_amd as st

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(args.warmup):
            b.copy_(a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / max(args.steps, 1)
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                          "steps": args.steps, "GBs": 2 * nbytes / dt / 1e9}), flush=True)
        return 0

    if args.op == "syev":
        return run_syev(args, torch, st)
    if args.workload in W.DENSE_WORKLOADS:
        print("bench.py: %s is a dense workload: use --op syev" % args.workload, file=sys.stderr)
        return 2
    w = W.WORKLOADS[args.workload or W.HEADLINE]
    jobz = args.jobz == "V"
    bt = bool(args.back_transform)
    if bt and not jobz:
        print("bench.py: --back-transform needs --jobz V", file=sys.stderr)
        return 2
    method = 1 if args.method == "bisect" else 0
    if method and jobz:
        print("bench.py: --method bisect needs --jobz N", file=sys.stderr)
        return 2
    scheme = 1 if args.scheme == "pg" else 0
    prm0 = st.make_params(lanes_per_problem=args.lanes, waves_per_block=args.waves,
                          band_storage=args.band, update_scheme=scheme, method=method)
    if args.batch < 0:
        print("bench.py: --batch must be positive", file=sys.stderr)
        return 2
    nb0 = args.batch or w.batch
    lanes0 = st.steqr_query(w.n, nb0, int(jobz), 0 if w.dtype == "f32" else 1,
                            prm0)["lanes_per_problem"]
    d, e = W.make_batch(w, nb0, replicate=max(1, 64 // lanes0) if args.replicate else 1)
    dev = torch.device("cuda:0")
    td = torch.from_numpy(d).to(dev)
    te = torch.from_numpy(e).to(dev)
    nb, n = d.shape
    lam = torch.empty_like(td)
    Q = torch.empty((nb, n, n), dtype=td.dtype, device=dev) if jobz else None
    Z = None
    if bt:
        # each step overwrites Q in place with Q times the rotations: the
        # basis stays orthogonal and its values do not change the work
        Z = W.random_basis(n, nb, d.dtype, salt=11)
        Q.copy_(torch.from_numpy(Z))
    info = torch.empty((nb,), dtype=torch.int32, device=dev)
    prm = st.make_params(lanes_per_problem=args.lanes, waves_per_block=args.waves,
                         band_storage=args.band, update_scheme=scheme, back_transform=bt,
                         method=method)
    plan = st.steqr_query(n, nb, int(jobz), st.dtype_code(td.dtype), prm)
    stream = torch.cuda.current_stream()

    def step():
        rc = st.steqr_batched_ex(td, te, lam, Q, n, nb, int(jobz), st.dtype_code(td.dtype),
                                 stream, info, prm)
        if rc != 0:
            raise st.SteqrError(rc, "steqr_batched_ex")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.max().item()) != 0 and np.isfinite(d).all():
        raise RuntimeError("non-convergence on a finite workload")

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps  # mean kernel duration (back-to-back launches)
    sec = ms / 1e3

    # spread: five short rounds of back-to-back launches
    rounds = []
    kr = max(5, args.steps // 10)
    for _ in range(5):
        start.record(stream)
        for _ in range(kr):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        rounds.append(start.elapsed_time(stop) / kr)
    spread = {"rounds": 5, "launches_per_round": kr, "ms_min": min(rounds),
              "ms_max": max(rounds)}

    # saturation: per-matrix time at twice the batch (the batch repeated)
    saturation = None
    if not args.replicate and not bt and not args.no_named and not args.no_saturation:
        td2 = torch.cat([td, td])
        te2 = torch.cat([te, te])
        lam2 = torch.empty_like(td2)
        Q2 = torch.empty((2 * nb, n, n), dtype=td.dtype, device=dev) if jobz else None
        info2 = torch.empty((2 * nb,), dtype=torch.int32, device=dev)
        # the same kernel: the default lanes per problem of values-only
        # launches depend on the batch, so fix the ones of the timed launch
        prm2 = st.make_params(lanes_per_problem=plan["lanes_per_problem"],
                              waves_per_block=args.waves,
                              band_storage=plan["band_storage"] if method == 0 else 0,
                              update_scheme=scheme, back_transform=bt, method=method)

        def step2():
            rc = st.steqr_batched_ex(td2, te2, lam2, Q2, n, 2 * nb, int(jobz),
                                     st.dtype_code(td.dtype), stream, info2, prm2)
            if rc != 0:
                raise st.SteqrError(rc, "steqr_batched_ex")
        step2()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(kr):
            step2()
        stop.record(stream)
        torch.cuda.synchronize()
        ms2 = start.elapsed_time(stop) / kr
        saturation = {"batch": 2 * nb, "ms_per_step": ms2,
                      "us_per_matrix_ratio_2x_over_1x": (ms2 / (2 * nb)) / (ms / nb)}
        del td2, te2, lam2, Q2, info2

    # secondary timing at the lanes-per-problem the workload list names
    named = None
    if (args.lanes == 0 and plan["lanes_per_problem"] != w.lanes and not args.replicate
            and not args.no_named and not method):
        prm_n = st.make_params(lanes_per_problem=w.lanes, waves_per_block=args.waves,
                               band_storage=1 if w.n <= 32 else 2, update_scheme=scheme,
                               back_transform=bt)
        try:
            st.steqr_query(n, nb, int(jobz), st.dtype_code(td.dtype), prm_n)
        except st.SteqrError:
            prm_n = None
        if prm_n is not None:
            def step_n():
                rc = st.steqr_batched_ex(td, te, lam, Q, n, nb, int(jobz),
                                         st.dtype_code(td.dtype), stream, info, prm_n)
                if rc != 0:
                    raise st.SteqrError(rc, "steqr_batched_ex")
            for _ in range(3):
                step_n()
            k = max(10, args.steps // 4)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(k):
                step_n()
            stop.record(stream)
            torch.cuda.synchronize()
            ms_n = start.elapsed_time(stop) / k
            named = {"lanes_per_problem": w.lanes, "ms_per_step": ms_n,
                     "value": nb / (ms_n / 1e3), "steps": k}

    cpu = None
    flops = None
    if not args.no_cpu:
        cpu, stats = cpu_baseline(d, e, jobz, w.name, scheme, Z, method)
        fin = np.isfinite(d).all(1) & np.isfinite(e).all(1)
        if method:
            flops = float(bisect_flops_per_matrix(stats[fin], n).sum())
        else:
            flops = float(flops_per_matrix(stats[fin], n, jobz).sum())
    dtype = w.dtype
    peak = PEAK_TFLOPS[dtype]
    roof = None
    family = kernel_family(plan, jobz, method)
    kname = kernel_label(plan, jobz, dtype, family, scheme)
    if flops is not None:
        ach = flops / sec / 1e12
        # the counter records are per launch of the workload's own batch
        ctr = (None if args.replicate or nb != w.batch
               else counters_from_profiles(w.name, jobz, family, kname,
                                           record_suffix(bt, scheme, method)))
        roof = {"kernel": kname,
                "bound": "alu", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak,
                # the published FP32 peak counts packed FP32 FMAs, which this
                # build does not emit (-packed-fp32-ops); the non-packed rate
                # is half of it (the FP64 peak is non-packed already)
                "peak_nonpacked": PEAK_NONPACKED_TFLOPS,
                "frac_nonpacked": ach / PEAK_NONPACKED_TFLOPS,
                "traffic": None if ctr is None else ctr.get("hbm_bytes_per_launch"),
                "algorithmic_flops_per_launch": flops,
                "algorithmic_flops_per_matrix": flops / nb}
        if ctr is not None and ctr.get("executed_flops_per_launch"):
            # executed VALU FLOPs (64 lanes x FP counter) at this run's time
            ex = ctr["executed_flops_per_launch"] / sec / 1e12
            roof["executed"] = {"tflops": ex, "frac": ex / peak,
                                "frac_nonpacked": ex / PEAK_NONPACKED_TFLOPS,
                                "flops_per_launch": ctr["executed_flops_per_launch"],
                                "source": "rocprofv3 SQ_INSTS_VALU_FLOPS_FP%s" % dtype[1:]}
        if ctr is not None and ctr.get("valu_insts_replicated"):
            roof["divergence"] = ctr["valu_insts_per_launch"] / ctr["valu_insts_replicated"]
        rv = (ctr or {}).get("raw", {}).get("valu")
        if rv and rv.get("SQ_BUSY_CYCLES") and rv.get("SQ_ACTIVE_INST_VALU"):
            # VALU busy: 4 cycles per wave64 instruction over every SIMD's
            # cycles (SQ_BUSY_CYCLES sums 32 shader engines); lane use: active
            # lanes per VALU instruction
            roof["valu_busy"] = rv["SQ_INSTS_VALU"] * 4.0 / (1024.0 * rv["SQ_BUSY_CYCLES"] / 32.0)
            roof["valu_lane_utilisation"] = (rv["SQ_THREAD_CYCLES_VALU"]
                                             / (64.0 * rv["SQ_ACTIVE_INST_VALU"]))
    bpm = bytes_per_matrix(n, d.itemsize, jobz, bt)
    out = {
        "metric": "matrices/sec (us/matrix) float n=16 jobz=V; % FP32 VALU peak",
        "value": nb / sec,
        "unit": "matrices/s",
        "us_per_matrix": sec / nb * 1e6,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n": n, "batch": nb, "jobz": "V" if jobz else "N",
                   "precision": dtype, "lanes_per_problem": plan["lanes_per_problem"],
                   "rows_per_lane": plan["rows_per_lane"], "padded_n": plan["padded_n"],
                   "band_storage": {1: "registers", 2: "LDS",
                                    3: "LDS, producer and consumer wavefronts"}[plan["band_storage"]],
                   "waves_per_block": plan["waves_per_block"],
                   "update_scheme": args.scheme.upper(),
                   "back_transform": bt,
                   "method": args.method.upper(),
                   "workgroups": plan["workgroups"],
                   "inputs": ("replicated per wavefront (lockstep ideal)" if args.replicate
                              else ("90% iid N(0,1) + 10% edge items" if w.edge_mix
                                    else "d,e iid N(0,1)")) + ", seed 1234"},
        "roofline": roof,
        "spread": spread,
        "saturation": saturation,
        "at_named_lanes": named,
        "hbm": {"algorithmic_bytes_per_launch": bpm * nb,
                "achieved_GBs": bpm * nb / sec / 1e9, "peak_GBs": HBM_PEAK_GBS},
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
        "library": st.version(),
    }
    print(json.dumps(out), flush=True)
    return 0


def dense_flops_per_matrix(n: int, jobz: bool) -> float:
    """Algorithmic flops of the dense front end: the reduction to tridiagonal
    form (4n^3/3) and, with eigenvectors, the formation of its Q (4n^3/3),
    the textbook counts (the kernel's full-storage form performs more)."""
    return (4.0 / 3.0) * n ** 3 * (2 if jobz else 1)


def run_syev(args, torch, st) -> int:
    """One step = one launch of syev_batched_ex over a dense workload."""
    name = args.workload or "s_f32_n16"
    if name not in W.DENSE_WORKLOADS:
        print("bench.py: --op syev needs a dense workload (%s)" % ", ".join(W.DENSE_WORKLOADS),
              file=sys.stderr)
        return 2
    dtype, n, nb = W.DENSE_WORKLOADS[name]
    if args.batch < 0:
        print("bench.py: --batch must be positive", file=sys.stderr)
        return 2
    nb = args.batch or nb
    jobz = args.jobz == "V"
    A = W.make_dense(name, nb)
    dev = torch.device("cuda:0")
    tA = torch.from_numpy(A).to(dev)
    lam = torch.empty((nb, n), dtype=tA.dtype, device=dev)
    Q = torch.empty_like(tA) if jobz else None
    info = torch.empty((nb,), dtype=torch.int32, device=dev)
    prm = st.make_params(lanes_per_problem=args.lanes, waves_per_block=args.waves)
    dcode = st.dtype_code(tA.dtype)
    plan = st.syev_query(n, nb, int(jobz), dcode, prm)
    stream = torch.cuda.current_stream()

    def step():
        rc = st.syev_batched_ex(tA, lam, Q, n, nb, int(jobz), dcode, stream, info, prm)
        if rc != 0:
            raise st.SteqrError(rc, "syev_batched_ex")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.max().item()) != 0:
        raise RuntimeError("non-convergence on a finite workload")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    sec = ms / 1e3

    cpu = None
    roof = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        oracle.syev(A[:64], jobz)
        times = []
        for _ in range(3):
            t = time.perf_counter()
            oracle.syev(A, jobz, threads=cores)
            times.append(time.perf_counter() - t)
        tmed = statistics.median(times)
        cpu = {"value": nb / tmed, "unit": "matrices/s", "cores": cores, "kind": "oracle",
               "us_per_matrix": tmed / nb * 1e6,
               "sample": "full %s batch (%d matrices), median of 3 runs on %d threads"
                         % (name, nb, cores)}
        # algorithmic flops: the dense front end plus the tridiagonal solve of
        # the reduced matrices (the oracle's rotation counts)
        d, e, _ = oracle.sytrd(A, want_q=False)
        _, _, _, stats = oracle.steqr(d, e, jobz, threads=cores)
        flops = float(flops_per_matrix(stats, n, jobz).sum()) + nb * dense_flops_per_matrix(n, jobz)
        ach = flops / sec / 1e12
        peak = PEAK_TFLOPS[dtype]
        roof = {"kernel": "steqr_%s_kernel<%s, N=%d, P=%d, %s, dense>"
                          % ("chunkl" if plan["band_storage"] == 2 else "chunk",
                             "float" if dtype == "f32" else "double", plan["padded_n"],
                             plan["lanes_per_problem"], "V" if jobz else "N"),
                "bound": "alu", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": None,
                "algorithmic_flops_per_launch": flops,
                "algorithmic_flops_per_matrix": flops / nb}
    itemsize = A.itemsize
    bpm = (n * n + n + (n * n if jobz else 0)) * itemsize
    out = {
        "metric": "matrices/sec (us/matrix) fused dense syev",
        "value": nb / sec,
        "unit": "matrices/s",
        "us_per_matrix": sec / nb * 1e6,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": name, "op": "syev", "n": n, "batch": nb,
                   "jobz": "V" if jobz else "N", "precision": dtype,
                   "lanes_per_problem": plan["lanes_per_problem"],
                   "rows_per_lane": plan["rows_per_lane"], "padded_n": plan["padded_n"],
                   "waves_per_block": plan["waves_per_block"],
                   "workgroups": plan["workgroups"],
                   "band_storage": {1: "registers", 2: "LDS"}[plan["band_storage"]],
                   "inputs": "dense symmetric, lower triangle iid N(0,1), seed 1234"},
        "roofline": roof,
        "hbm": {"algorithmic_bytes_per_launch": bpm * nb,
                "achieved_GBs": bpm * nb / sec / 1e9, "peak_GBs": HBM_PEAK_GBS},
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
        "library": st.version(),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
