"""Per-launch hardware-counter record of a workload's default kernel.

Runs bench.py under rocprofv3 once per counter group (the hardware collects
a limited number of counters per pass) and writes
profiles/counters_<workload>_<V|N>.json, which bench.py reads to report the
HBM traffic, the executed VALU FLOP rate, VALU busy and the divergence from
the lockstep ideal next to its timing. Run on the GPU machine from the
repository root, e.g.

    python3 profile_counters.py --calibrate c2_f32_n16:V c3_f64_n12:V

Counter groups (one rocprofv3 --pmc pass each):
  fetch / write     FETCH_SIZE, WRITE_SIZE (KiB per dispatch), scaled by what
                    the same counters read for a plain device copy / fill of
                    256 MiB (--calibrate; else the factors of an earlier record);
  valu              SQ_WAVES, SQ_INSTS_VALU, SQ_INSTS_SALU, SQ_INSTS_LDS,
                    SQ_ACTIVE_INST_VALU, SQ_THREAD_CYCLES_VALU, SQ_WAVE_CYCLES,
                    SQ_BUSY_CYCLES;
  valu_replicated   the same on the replicated batch (every chunk of a
                    wavefront holds the same matrix: the lockstep ideal);
  flops             SQ_INSTS_VALU_FLOPS_FP32/64 and its parts (FMA, MUL, ADD,
                    TRANS), SQ_INSTS_VALU_INT32, SQ_INSTS_VALU_CVT,
                    SQ_INSTS_VALU.
The record holds the median over the profiled dispatches of the solver's
kernel and the exact commands.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import statistics
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

VALU_GROUP = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU",
              "SQ_THREAD_CYCLES_VALU", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"]


def flops_group(prec: str):
    b = "F32" if prec == "f32" else "F64"
    return ["SQ_INSTS_VALU_FLOPS_FP%s" % b[1:], "SQ_INSTS_VALU_FMA_%s" % b,
            "SQ_INSTS_VALU_MUL_%s" % b, "SQ_INSTS_VALU_ADD_%s" % b, "SQ_INSTS_VALU_TRANS_%s" % b,
            "SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU"]


def run_pass(counters, bench_args, kernel_key: str, timeout: int):
    """One rocprofv3 pass; returns ({counter: median per dispatch}, median
    dispatch microseconds, number of dispatches, the command)."""
    out = tempfile.mkdtemp(prefix="ctr_", dir=os.environ.get("TMPDIR", "/tmp"))
    cmd = ["timeout", "-s", "KILL", str(timeout), "rocprofv3", "--pmc", *counters, "-d", out,
           "-o", "run", "--output-format", "csv", "--", "python3", "bench.py", *bench_args]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    files = glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True)
    if r.returncode != 0 and not files:
        shutil.rmtree(out, ignore_errors=True)
        raise RuntimeError("rocprofv3 failed (rc %d): %s\n%s" % (r.returncode, " ".join(cmd),
                                                                r.stderr[-2000:]))
    per = {}   # dispatch id -> {counter: value}
    dur = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kernel_key not in row.get("Kernel_Name", ""):
                    continue
                did = row.get("Dispatch_Id") or row.get("Correlation_Id")
                per.setdefault(did, {})[row["Counter_Name"]] = float(row["Counter_Value"])
                try:
                    dur[did] = (float(row["End_Timestamp"]) - float(row["Start_Timestamp"])) / 1e3
                except (KeyError, ValueError):
                    pass
    shutil.rmtree(out, ignore_errors=True)
    if not per:
        raise RuntimeError("no dispatch of %r in %s" % (kernel_key, " ".join(cmd)))
    vals = {c: statistics.median(d[c] for d in per.values() if c in d)
            for c in counters if any(c in d for d in per.values())}
    us = statistics.median(dur.values()) if dur else None
    return vals, us, len(per), " ".join(cmd[4:]).replace(out, "OUT")


# launch option sets with records of their own (case "workload:J:mode")
MODE_ARGS = {"bt": ["--back-transform"], "pg": ["--scheme", "pg"], "bisect": ["--method", "bisect"]}


def kernel_family(st, wname: str, jobz: bool, mode: str = ""):
    import workloads as W
    w = W.WORKLOADS[wname]
    import bench
    scheme, method = int(mode == "pg"), int(mode == "bisect")
    plan = st.steqr_query(w.n, w.batch, int(jobz), 0 if w.dtype == "f32" else 1,
                          st.make_params(update_scheme=scheme, method=method))
    fam = bench.kernel_family(plan, jobz, method)
    return fam, bench.kernel_label(plan, jobz, w.dtype, fam, scheme), w


def calibrate(timeout: int) -> dict:
    mib = 256
    args = ["--copy-calibration", str(mib), "--steps", "3", "--warmup", "1"]
    f, _, _, c1 = run_pass(["FETCH_SIZE"], args, "copyBuffer", timeout)
    w, _, _, c2 = run_pass(["WRITE_SIZE"], args, "Fill", timeout)
    nbytes = mib << 20
    return {"fetch_factor": nbytes / (f["FETCH_SIZE"] * 1024.0),
            "write_factor": nbytes / (w["WRITE_SIZE"] * 1024.0),
            "reference": "%d MiB device copy (copyBuffer kernel) read for FETCH_SIZE, %d MiB "
                         "fill written for WRITE_SIZE" % (mib, mib),
            "raw": {"copy_FETCH_SIZE_KiB": f["FETCH_SIZE"], "fill_WRITE_SIZE_KiB": w["WRITE_SIZE"]},
            "commands": [c1, c2]}


def collect(wname: str, jobz: bool, cal: dict, timeout: int, mode: str = "") -> dict:
    import bench
    import symmetric_tridiagonal_eigensolver_amd as st
    fam, kname, w = kernel_family(st, wname, jobz, mode)
    key = "steqr_%s_kernel" % fam
    base = ["--workload", wname, "--jobz", "V" if jobz else "N", "--steps", "3", "--warmup", "1",
            "--no-cpu", "--no-named", "--no-saturation"] + MODE_ARGS.get(mode, [])
    raw, cmds = {}, []
    for tag, ctrs, extra in (("fetch", ["FETCH_SIZE"], []), ("write", ["WRITE_SIZE"], []),
                             ("valu", VALU_GROUP, []), ("valu_replicated", VALU_GROUP, ["--replicate"]),
                             ("flops", flops_group(w.dtype), [])):
        t = time.time()
        vals, us, nd, cmd = run_pass(ctrs, base + extra, key, timeout)
        vals["dur_us"] = us
        raw[tag] = vals
        cmds.append(cmd)
        print("  %s %s %s: %d dispatches, %.1fs" % (wname, "V" if jobz else "N", tag, nd,
                                                   time.time() - t), flush=True)
    fetch = raw["fetch"]["FETCH_SIZE"] * 1024.0 * cal["fetch_factor"]
    write = raw["write"]["WRITE_SIZE"] * 1024.0 * cal["write_factor"]
    fl = raw["flops"]
    fc = "SQ_INSTS_VALU_FLOPS_FP%s" % ("32" if w.dtype == "f32" else "64")
    return {
        "workload": wname, "jobz": "V" if jobz else "N", "mode": mode, "kernel": kname,
        "kernel_source_hash": bench.kernel_source_hash(fam),
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
        "hbm_bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": bench.bytes_per_matrix(w.n, 4 if w.dtype == "f32" else 8,
                                                               jobz, mode == "bt") * w.batch,
        "calibration": {k: cal[k] for k in ("fetch_factor", "write_factor", "reference")},
        "valu_insts_per_launch": raw["valu"]["SQ_INSTS_VALU"],
        "salu_insts_per_launch": raw["valu"]["SQ_INSTS_SALU"],
        "valu_insts_replicated": raw["valu_replicated"]["SQ_INSTS_VALU"],
        "salu_insts_replicated": raw["valu_replicated"]["SQ_INSTS_SALU"],
        "executed_flops_per_launch": 64.0 * fl.get(fc, 0.0),
        "flops_counter": fc,
        "profiled_dispatch_us": raw["valu"]["dur_us"],
        "commands": cal.get("commands", []) + cmds,
        "raw": raw,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("cases", nargs="+",
                    help="workload:V or workload:N, optionally :bt, :pg or :bisect")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the copy / fill scale factors (else reuse the headline record's)")
    ap.add_argument("--timeout", type=int, default=120, help="seconds per rocprofv3 pass")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"),
                    help="directory for the records (default profiles/)")
    args = ap.parse_args()
    os.environ.setdefault("TMPDIR", "/tmp")
    if args.calibrate:
        cal = calibrate(args.timeout)
        print("calibration: fetch x%.4f write x%.4f" % (cal["fetch_factor"], cal["write_factor"]),
              flush=True)
    else:
        ref = json.load(open(os.path.join(ROOT, "profiles", "counters_c2_f32_n16_V.json")))
        cal = dict(ref["calibration"])
    import bench
    for case in args.cases:
        parts = case.split(":")
        wname, j, mode = parts[0], parts[1], (parts[2] if len(parts) > 2 else "")
        rec = collect(wname, j == "V", cal, args.timeout, mode)
        os.makedirs(args.out, exist_ok=True)
        suffix = bench.record_suffix(mode == "bt", int(mode == "pg"), int(mode == "bisect"))
        path = os.path.join(args.out, "counters_%s_%s%s.json" % (wname, j, suffix))
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print("wrote %s: VALU %.3g, divergence %.3f, HBM %.4g B (algorithmic %.4g)" % (
            path, rec["valu_insts_per_launch"],
            rec["valu_insts_per_launch"] / rec["valu_insts_replicated"],
            rec["hbm_bytes_per_launch"], rec["algorithmic_bytes_per_launch"]), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
