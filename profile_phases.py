"""Where a default kernel's time goes: per-wavefront phase cycles, and the
latency of dependent operations.

The kernels mark their phases with STEQR_PHASE_* statements, which expand to
nothing in libsteqr.so. This script builds the profiling library
(probes/steqr_phase_probe.hip, the same kernel templates with the timers
compiled in) and, on the GPU, launches each case's kernel with the launch
shape the library's default plan gives the workload, checks that its
results equal the library's bit for bit, and writes a summary per case:

    python3 profile_phases.py --build-only          # on the build machine
    python3 profile_phases.py --out OUT                   # on an MI355X

Slots (cycles of the shader clock read with s_memtime, added up between
consecutive marks, per wavefront):
  chunked kernel          0 load, 5 settle up to the next operation (block
                          opens, deflation scan, masks), 6 settle's closes
                          and shift, 1 settle's 2x2 setup, 2 chase, 3
                          epilogue (final closes, sort, stores), 4 passes;
  producer-consumer       producer: 0 load, 1 settle, 2 chase, 3 epilogue,
                          4 waiting for the consumers at the end of a pass,
                          5 passes, 6 sum of the chase bounds;
                          consumers: 0 load, 1 waiting for a pass, 2 applying
                          a pass, 3 epilogue (sorted store of Q), 5 passes;
  both                    7, 8 the wavefront's start and end times on the
                          constant 100 MHz counter (s_memrealtime).
The latency kernels time chains of 4096 dependent operations in one
wavefront and measure the shader clock counter's rate.
"""
from __future__ import annotations

import argparse
import ctypes as ct
import os
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PKG = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd")
PROBE_SRC = os.path.join(PKG, "probes", "steqr_phase_probe.hip")
PROBE_LIB = os.path.join(PKG, "probes", "libsteqr_phase.so")

# case -> (probe kernel index, dtype, padded order, lanes per problem, band
# storage, consumer wavefronts per workgroup or 0)
CASES = {
    "c2_f32_n16:V": (0, "f32", 16, 4, 1, 0),
    "c5_f64_n64:V": (1, "f64", 64, 4, 3, 11),
    "w_f64_n128:V": (2, "f64", 128, 32, 3, 8),
    "w_f32_n128:V": (3, "f32", 128, 8, 3, 10),
    "c2_f32_n16:N": (4, "f32", 16, 2, 1, 0),
    "c4_f64_n32:N": (5, "f64", 32, 1, 1, 0),
    "w_f32_n256:V": (6, "f32", 256, 64, 3, 8),
    "w_f64_n256:V": (7, "f64", 256, 64, 3, 8),
    "w_f32_n512:V": (8, "f32", 512, 64, 3, 8),
    "w_f64_n512:V": (9, "f64", 512, 64, 3, 8),
}
LATENCY = ["double FMA (v_fma_f64)", "double reciprocal square root (v_rsq_f64)",
           "refined double reciprocal square root (solver's rsq_refined)",
           "float FMA (v_fma_f32)", "float reciprocal square root (v_rsq_f32)"]
LATENCY_ITERS = 256  # x 16 operations
SLOTS = 9  # per-wavefront slots the profiling build stores


def probe_build_command():
    """hipcc command of the profiling library (the library's own flags)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_steqr_build", os.path.join(PKG, "build.py"))
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)
    return [B.HIPCC, *B.HIP_FLAGS, "-shared", "-o", PROBE_LIB, PROBE_SRC]


def build_probe() -> str:
    r = subprocess.run(probe_build_command(), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed:\n%s" % r.stderr)
    return PROBE_LIB


def load_probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("%s is not built (python3 profile_phases.py --build-only)" % PROBE_LIB)
    lib = ct.CDLL(PROBE_LIB)
    lib.steqr_phase_launch.restype = ct.c_int
    lib.steqr_phase_launch.argtypes = [ct.c_int] + [ct.c_void_p] * 5 + [ct.c_int] * 4 + [
        ct.c_void_p, ct.c_void_p]
    lib.steqr_latency_launch.restype = ct.c_int
    lib.steqr_latency_launch.argtypes = [ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p,
                                         ct.c_void_p]
    lib.steqr_seed_launch.restype = ct.c_int
    lib.steqr_seed_launch.argtypes = [ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_int, ct.c_void_p]
    return lib


SEED_COUNT = 1 << 22


def seeds(torch, lib):
    """Worst relative error of the double reciprocal and reciprocal square
    root seeds (v_rcp_f64, v_rsq_f64) over SEED_COUNT seeded inputs with
    mantissas uniform in [1, 2) and exponents uniform in -900..900 (either
    sign for the reciprocal), against long double on the host."""
    import numpy as np
    g = np.random.default_rng(20261203)
    m = 1.0 + g.random(SEED_COUNT)
    ex = g.integers(-900, 901, SEED_COUNT)
    x = np.ldexp(m, ex)
    rows = []
    for kind, name in ((0, "reciprocal (v_rcp_f64)"), (1, "reciprocal square root (v_rsq_f64)")):
        xs = np.where(np.arange(SEED_COUNT) % 2 == 1, -x, x) if kind == 0 else x
        tx = torch.from_numpy(xs).cuda()
        ty = torch.empty_like(tx)
        rc = lib.steqr_seed_launch(kind, tx.data_ptr(), ty.data_ptr(), SEED_COUNT,
                                   torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("seed launch failed: %d" % rc)
        torch.cuda.synchronize()
        y = ty.cpu().numpy().astype(np.longdouble)
        xl = xs.astype(np.longdouble)
        exact = 1.0 / xl if kind == 0 else 1.0 / np.sqrt(xl)
        rel = np.abs((y - exact) / exact)
        k = int(np.argmax(rel))
        rows.append((name, float(rel[k]), float(np.log2(float(rel[k]))), float(xs[k])))
    return rows


def write_seeds(rows, out: str, command: str) -> str:
    lines = ["# Accuracy of the double reciprocal and reciprocal square root seeds", "",
             "Command (repository root, MI355X): `%s`" % command, "",
             "%d seeded inputs per row (mantissas uniform in [1, 2), exponents uniform in "
             "-900..900, alternate signs for the reciprocal), each seed against the exact "
             "value in long double on the host. The solver refines the reciprocal square "
             "root and, in the bisection's Sturm count, the reciprocal by one third-order step, "
             "whose error is the cube of the seed's." % SEED_COUNT, "",
             "| seed | worst relative error | log2 | at x |", "|---|---:|---:|---:|"]
    lines += ["| %s | %.3e | %.2f | %.17g |" % r for r in rows]
    path = os.path.join(out, "seed_accuracy.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def kernel_ms(torch, fn, reps: int = 5) -> float:
    """Median of `reps` event-timed launches on the current stream."""
    s = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return statistics.median(out)


def profile_case(torch, lib, case: str) -> dict:
    import numpy as np
    import symmetric_tridiagonal_eigensolver_amd as st
    import workloads as W
    which, dt, N, P, band, nc = CASES[case]
    wname, j = case.split(":")
    jobz = j == "V"
    w = W.WORKLOADS[wname]
    dcode = st.STEQR_F32 if w.dtype == "f32" else st.STEQR_F64
    plan = st.steqr_query(w.n, w.batch, int(jobz), dcode)
    want = {"padded_n": N, "lanes_per_problem": P, "band_storage": band}
    got = {k: plan[k] for k in want}
    if got != want or w.dtype != dt or (nc and plan["waves_per_block"] != nc + 1):
        raise RuntimeError("%s: the library's default plan %s is not the probe's kernel %s"
                           % (case, plan, want))
    d, e = W.make_batch(w)
    td = torch.from_numpy(d).cuda()
    te = torch.from_numpy(e).cuda()
    B, n = d.shape
    lam = torch.empty_like(td)
    Q = torch.empty((B, n, n) if jobz else (1,), dtype=td.dtype, device="cuda")
    info = torch.empty(B, dtype=torch.int32, device="cuda")
    lam2, Q2, info2 = torch.empty_like(lam), torch.empty_like(Q), torch.empty_like(info)
    grid, block = plan["workgroups"], plan["waves_per_block"] * 64
    nwaves = grid * plan["waves_per_block"]
    ph = torch.zeros((nwaves, SLOTS), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def probe():
        rc = lib.steqr_phase_launch(which, td.data_ptr(), te.data_ptr(), lam.data_ptr(),
                                    Q.data_ptr() if jobz else None, info.data_ptr(), n, B, grid,
                                    block, ph.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError("probe launch failed: %d" % rc)

    def product():
        rc = st.steqr_batched_ex(td, te, lam2, Q2 if jobz else None, n, B, int(jobz), dcode,
                                 info=info2)
        if rc != 0:
            raise RuntimeError("library launch failed: %d" % rc)

    probe()
    product()
    torch.cuda.synchronize()
    # bit for bit (NaN items of the edge mixes included)
    it = torch.int32 if td.dtype == torch.float32 else torch.int64
    same = (torch.equal(lam.view(it), lam2.view(it))
            and (not jobz or torch.equal(Q.view(it), Q2.view(it))) and torch.equal(info, info2))
    if not same:
        raise RuntimeError("%s: the timed kernel's results differ from the library's" % case)
    t_probe = kernel_ms(torch, probe)
    t_prod = kernel_ms(torch, product)
    a = ph.cpu().numpy().astype(np.float64)
    res = {"case": case, "workload": wname, "n": n, "batch": B, "plan": plan,
           "probe_ms": t_probe, "library_ms": t_prod, "bit_equal": same}
    if nc == 0:
        tot = a[:, [0, 1, 2, 3, 5, 6]].sum(1)
        res["roles"] = {"wavefront": summarise(a, tot, passes_slot=4)}
        res["positions_per_pass"] = N - 1
        res["timeline"] = timeline(a)
    else:
        role = np.arange(nwaves) % (nc + 1)
        prod, cons = a[role == nc], a[role < nc]
        res["roles"] = {"producer": summarise(prod, prod[:, [0, 1, 2, 3, 4]].sum(1), 5),
                        "consumer": summarise(cons, cons[:, :4].sum(1), 5)}
        res["chase_bound_per_pass"] = float(prod[:, 6].sum() / max(prod[:, 5].sum(), 1))
        res["timeline"] = timeline(a)
    return res


def summarise(a, tot, passes_slot: int) -> dict:
    import numpy as np
    q = np.percentile(tot, [0, 50, 90, 100])
    return {"waves": int(a.shape[0]), "total_cycles": float(tot.mean()),
            "slots": [float(x) for x in a.mean(0)],
            "passes": float(a[:, passes_slot].mean()),
            "passes_max": float(a[:, passes_slot].max()),
            "lifetime_pct": [float(x) for x in q]}


def timeline(a) -> dict:
    """Start skew and span of the launch's wavefronts in microseconds (slots
    7 and 8: start and end on the 100 MHz counter)."""
    import numpy as np
    t0 = a[:, 7].min()
    start, end = (a[:, 7] - t0) / 100.0, (a[:, 8] - t0) / 100.0
    return {"start_skew": float(start.max()), "span": float(end.max()),
            "end_p50": float(np.median(end)), "end_min": float(end.min())}


def latency(torch, lib):
    """[(operation, cycles per dependent operation)], and the shader clock
    counter's rate in MHz (its advance over the constant 100 MHz counter's
    over the same chains)."""
    out = torch.empty(64, dtype=torch.float64, device="cuda")
    cyc = torch.zeros(2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rows, rates = [], []
    for k, name in enumerate(LATENCY):
        best = None
        for _ in range(3):
            rc = lib.steqr_latency_launch(k, LATENCY_ITERS, out.data_ptr(), cyc.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError("latency launch failed: %d" % rc)
            torch.cuda.synchronize()
            t, r = (int(v) for v in cyc.cpu().tolist())
            c = t / (16.0 * LATENCY_ITERS)
            best = c if best is None else min(best, c)
            if r > 0:
                rates.append(100.0 * t / r)
        rows.append((name, best))
    return rows, statistics.median(rates) if rates else None


ORDER = {"wavefront": [0, 5, 6, 1, 2, 3], "producer": [0, 1, 2, 4, 3], "consumer": [0, 1, 2, 3]}
PHASE_NAMES = {
    "wavefront": ["load", "settle: 2x2 setup", "chase", "epilogue", None,
                  "settle: opens, scan, masks", "settle: closes, shift"],
    "producer": ["load", "settle", "chase", "epilogue", "wait for consumers"],
    "consumer": ["load", "wait for a pass", "apply a pass", "epilogue (store)"],
}


def write_case(res: dict, out: str, command: str, mhz) -> str:
    case = res["case"]
    wname, j = case.split(":")
    p = res["plan"]
    lines = ["# Phase cycles: %s, jobz = %s" % (wname, j), "",
             "Command (repository root, MI355X): `%s`" % command, "",
             "Kernel: the library's default launch for order %d, batch %d (padded order %d, "
             "%d lanes per problem, band storage %d, %d wavefronts per workgroup, %d "
             "workgroups). The profiling build's results equal the library's bit for bit."
             % (res["n"], res["batch"], p["padded_n"], p["lanes_per_problem"],
                p["band_storage"], p["waves_per_block"], p["workgroups"]), "",
             "Kernel time: %.1f us with the timers, %.1f us without (library). Cycles are "
             "those of the shader clock counter (s_memtime), which advanced at %s over the "
             "latency chains of the same run." % (
                 res["probe_ms"] * 1e3, res["library_ms"] * 1e3,
                 "%.0f MHz" % mhz if mhz else "an unmeasured rate"), ""]
    for role, s in res["roles"].items():
        names = PHASE_NAMES[role]
        tot = s["total_cycles"]
        lines += ["## %s (%d wavefronts; mean per wavefront)" % (role, s["waves"]), "",
                  "| phase | cycles | share | per pass |", "|---|---:|---:|---:|"]
        for k in ORDER[role]:
            nm = names[k]
            c = s["slots"][k]
            per = c / s["passes"] if s["passes"] and k in (1, 2, 4, 5, 6) else None
            lines.append("| %s | %.0f | %.1f%% | %s |" % (nm, c, 100 * c / tot,
                                                          "%.0f" % per if per else ""))
        lq = s["lifetime_pct"]
        lines += ["| total | %.0f | | |" % tot, "",
                  "Passes per wavefront: mean %.1f, max %.0f. Wavefront lifetime (cycles): "
                  "min %.0f, median %.0f, 90th percentile %.0f, max %.0f%s." % (
                      s["passes"], s["passes_max"], lq[0], lq[1], lq[2], lq[3],
                      " (mean %.1f us, max %.1f us)" % (tot / mhz, lq[3] / mhz) if mhz else ""),
                  ""]
        if role == "wavefront":
            lines.append("Chase cycles per position (%d positions per pass): %.1f."
                         % (res["positions_per_pass"],
                            s["slots"][2] / s["passes"] / res["positions_per_pass"]))
            lines.append("")
        if role == "producer":
            cb = res["chase_bound_per_pass"]
            lines.append("Mean chase bound (positions the wavefront's chase runs to) per pass: "
                         "%.1f; chase cycles per position: %.0f." % (cb, s["slots"][2] / s["passes"] / cb))
            lines.append("")
    tl = res["timeline"]
    lines += ["Timeline of all wavefronts (s_memrealtime, microseconds after the first "
              "start): the last started at %.1f; the first ended at %.1f, the median at "
              "%.1f, the last at %.1f." % (tl["start_skew"], tl["end_min"], tl["end_p50"],
                                            tl["span"]), ""]
    path = os.path.join(out, "phases_%s_%s.md" % (wname, j))
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def write_latency(rows, mhz, out: str, command: str) -> str:
    lines = ["# Dependent-operation latency (one wavefront)", "",
             "Command (repository root, MI355X): `%s`" % command, "",
             "Each row: %d dependent operations of one kind in a single wavefront, timed with "
             "s_memtime; best of three launches. The counter advanced at %s (against "
             "s_memrealtime's constant 100 MHz)." % (16 * LATENCY_ITERS,
                                                     "%.0f MHz" % mhz if mhz else "?"), "",
             "| operation | cycles per dependent operation |", "|---|---:|"]
    lines += ["| %s | %.1f |" % (nm, c) for nm, c in rows]
    path = os.path.join(out, "latency_dependent_chains.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("cases", nargs="*", default=list(CASES), help="workload:V or workload:N cases")
    ap.add_argument("--build-only", action="store_true", help="build the probe library and exit")
    ap.add_argument("--seeds", action="store_true",
                    help="only the accuracy of the double reciprocal seeds")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    if args.build_only:
        print("built", build_probe(), flush=True)
        return 0
    import torch
    if not torch.cuda.is_available():
        print("profile_phases.py needs a GPU", file=sys.stderr)
        return 1
    lib = load_probe()
    os.makedirs(args.out, exist_ok=True)
    if args.seeds:
        command = "python3 profile_phases.py --build-only && python3 profile_phases.py --seeds"
        print("  wrote", write_seeds(seeds(torch, lib), args.out, command), flush=True)
        return 0
    command = "python3 profile_phases.py --build-only && python3 profile_phases.py " + \
        " ".join(args.cases)
    print("latency chains", flush=True)
    rows, mhz = latency(torch, lib)
    print("  wrote", write_latency(rows, mhz, args.out, command), flush=True)
    for case in args.cases:
        print("phase case", case, flush=True)
        res = profile_case(torch, lib, case)
        print("  wrote", write_case(res, args.out, command, mhz), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
