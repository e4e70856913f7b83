"""Kernel traces and bench lines of every workload, and their summaries.

Per case (workload:V or workload:N), on an MI355X from the repository root:
  1. bench.py at the default launch (HIP-event mean over the timed region,
     roofline with the counter record's figures, CPU oracle baseline);
  2. rocprofv3 --kernel-trace --stats of the same bench.py command without
     its CPU, saturation and named-lanes legs, from which the solver
     kernel's dispatch statistics are taken.
Each case's results go to OUT/<workload>_<V|N>.json; `--summarise` turns the
JSON files of a directory into profiles/steqr_all_workloads_trace.md and the
headline's profiles/steqr_chunk_f32_n16_V_headline.md:

    python3 profile_workloads.py --out OUT c2_f32_n16:V c5_f64_n64:V ...
    python3 profile_workloads.py --summarise OUT
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CASES = ["c1_f32_n4:V", "c2_f32_n8:V", "c2_f32_n8:N", "c2_f32_n16:V", "c2_f32_n16:N",
         "c3_f64_n12:V", "c3_f64_n16:V", "c4_f32_n32:V", "c4_f32_n32:N", "c4_f64_n32:V",
         "c4_f64_n32:N", "c5_f64_n64:V", "c5_f64_n64:N", "w_f32_n128:V", "w_f32_n128:N",
         "w_f64_n128:V", "w_f64_n128:N", "w_f32_n256:V", "w_f32_n256:N", "w_f64_n256:V",
         "w_f64_n256:N", "w_f32_n512:V", "w_f32_n512:N", "w_f64_n512:V", "w_f64_n512:N"]
HEADLINE = "c2_f32_n16:V"

# The NEXT rows' option sets: case "workload:jobz:mode" with mode bt
# (back-transformation), syev (fused dense syev on a dense workload) or
# bisect (values-only bisection); each set has a summary of its own.
MODES = {"bt": ["--back-transform"], "syev": ["--op", "syev"], "bisect": ["--method", "bisect"],
         "pg": ["--scheme", "pg"]}
EXTRA_SETS = {
    "bt": ("steqr_back_transform.md", "Back-transformation (Q holds a basis on entry)",
           ["c2_f32_n16:V:bt", "c3_f64_n16:V:bt", "c4_f32_n32:V:bt", "c4_f64_n32:V:bt",
            "c5_f64_n64:V:bt", "w_f64_n128:V:bt"]),
    "syev": ("syev_chunk_dense_workloads.md",
             "Fused dense syev (reduction + tridiagonal solve + back-transformation)",
             ["s_f32_n8:V:syev", "s_f32_n8:N:syev", "s_f32_n16:V:syev", "s_f32_n16:N:syev",
              "s_f32_n32:V:syev", "s_f32_n32:N:syev", "s_f64_n16:V:syev", "s_f64_n16:N:syev",
              "s_f64_n32:V:syev", "s_f64_n32:N:syev"]),
    "pg": ("steqr_pg_step.md", "The Parlett-Gray form of the chase step",
           ["c2_f32_n16:V:pg", "c3_f64_n16:V:pg", "c4_f64_n32:V:pg", "c5_f64_n64:V:pg"]),
    "bisect": ("steqr_bisect_values.md", "Values-only bisection (steqr_bisect_kernel)",
               ["c2_f32_n8:N:bisect", "c2_f32_n16:N:bisect", "c4_f32_n32:N:bisect",
                "c3_f64_n16:N:bisect", "c4_f64_n32:N:bisect", "c5_f64_n64:N:bisect",
                "w_f32_n128:N:bisect", "w_f64_n128:N:bisect", "w_f32_n256:N:bisect",
                "w_f64_n256:N:bisect", "w_f32_n512:N:bisect", "w_f64_n512:N:bisect"]),
}


def split_case(case: str):
    parts = case.split(":")
    return parts[0], parts[1], (parts[2] if len(parts) > 2 else "")


def case_file(case: str) -> str:
    wname, j, mode = split_case(case)
    return "%s_%s%s.json" % (wname, j, "_" + mode if mode else "")


def bench_args(wname: str, j: str, mode: str = ""):
    steps = ("5" if wname.endswith("n512") else "20") if wname.startswith(("w_", "c5_")) else "200"
    return (["--workload", wname, "--jobz", j, "--steps", steps, "--warmup", "5"]
            + MODES.get(mode, []))


def trace_args(wname: str, j: str, mode: str = ""):
    # the bench line's own steps and warm-up, without the legs that launch
    # other shapes (twice the batch, other lanes) under the same kernel name
    return bench_args(wname, j, mode) + ["--no-cpu", "--no-named", "--no-saturation"]


def run_bench(args, timeout: int) -> dict:
    r = subprocess.run(["timeout", "-k", "10", str(timeout), sys.executable, "bench.py", *args],
                       cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("bench.py %s failed (rc %d): %s" % (" ".join(args), r.returncode,
                                                              r.stderr[-2000:]))
    return json.loads(r.stdout.strip().splitlines()[-1])


def run_trace(args, timeout: int):
    """rocprofv3 kernel-trace statistics of one bench.py run: list of
    {name, calls, avg_us, min_us, max_us, total_us}, and the command."""
    out = tempfile.mkdtemp(prefix="trace_", dir=os.environ.get("TMPDIR", "/tmp"))
    cmd = ["timeout", "-s", "KILL", str(timeout), "rocprofv3", "--kernel-trace", "--stats",
           "-d", out, "-o", "run", "--output-format", "csv", "--", "python3", "bench.py", *args]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    files = glob.glob(os.path.join(out, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        shutil.rmtree(out, ignore_errors=True)
        raise RuntimeError("rocprofv3 wrote no kernel statistics (rc %d): %s\n%s"
                           % (r.returncode, " ".join(cmd), r.stderr[-2000:]))
    rows = []
    with open(files[0]) as f:
        rd = csv.DictReader(f)
        cols = {c.lower(): c for c in (rd.fieldnames or [])}

        def col(*names):
            for nm in names:
                if nm in cols:
                    return cols[nm]
            raise RuntimeError("unexpected kernel statistics columns %s" % rd.fieldnames)
        cn, cc = col("name", "kernelname", "kernel_name"), col("calls")
        ct, ca = col("totaldurationns"), col("averagens")
        cmin, cmax = col("minns"), col("maxns")
        for row in rd:
            rows.append({"name": row[cn], "calls": int(row[cc]),
                         "total_us": float(row[ct]) / 1e3, "avg_us": float(row[ca]) / 1e3,
                         "min_us": float(row[cmin]) / 1e3, "max_us": float(row[cmax]) / 1e3})
    shutil.rmtree(out, ignore_errors=True)
    return rows, " ".join(cmd[4:]).replace(out, "OUT")


def solver_row(rows, family: str):
    key = "steqr_%s_kernel" % family
    cand = [r for r in rows if key in r["name"]]
    if not cand:
        raise RuntimeError("no %s in the trace" % key)
    return max(cand, key=lambda r: r["calls"])


def collect(case: str, out: str, timeout: int) -> str:
    wname, j, mode = split_case(case)
    t = time.time()
    line = run_bench(bench_args(wname, j, mode), timeout)
    print("  %s: bench.py done (%.0fs)" % (case, time.time() - t), flush=True)
    rows, tcmd = run_trace(trace_args(wname, j, mode), timeout)
    fam = line["roofline"]["kernel"].split("<")[0][len("steqr_"):-len("_kernel")]
    rec = {"case": case, "bench": line, "bench_command": "python3 bench.py " +
           " ".join(bench_args(wname, j, mode)), "trace": rows, "trace_command": tcmd,
           "solver": solver_row(rows, fam)}
    path = os.path.join(out, case_file(case))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print("  %s: %.1f us (trace %.1f us), %.0fs" % (case, line["ms_per_step"] * 1e3,
                                                   rec["solver"]["avg_us"], time.time() - t),
          flush=True)
    return path


def fmt(x, spec="%.3f"):
    return "—" if x is None else spec % x


def summarise(src: str) -> None:
    recs = {}
    for p in glob.glob(os.path.join(src, "*.json")):
        r = json.load(open(p))
        if "bench" in r:
            recs[r["case"]] = r
    order = [c for c in CASES if c in recs]
    if not order and HEADLINE not in recs and not any(
            c in recs for _, (_, _, cs) in EXTRA_SETS.items() for c in cs):
        raise SystemExit("no records in %s" % src)
    lines = [
        "# Kernel traces and bench lines of every workload (one MI355X)", "",
        "Per case (workload and jobz), bench.py at the default launch (HIP-event mean over the "
        "timed region, seeded synthetic inputs, recipes in workloads.py) and a rocprofv3 "
        "kernel-trace run of the same bench.py command, both from:", "",
        "    python3 profile_workloads.py --out OUT " + " ".join(order),
        "    python3 profile_workloads.py --summarise OUT", "",
        "which runs, per case:", "",
        "    python3 bench.py --workload WL --jobz J --steps S --warmup 5   (S = 5 at order 512, 20 for c5 and the other w_*, else 200)",
        "    rocprofv3 --kernel-trace --stats -d OUT -o run --output-format csv -- python3 bench.py --workload WL "
        "--jobz J --steps S --warmup 5 --no-cpu --no-named --no-saturation", "",
        "The trace average covers the warm-up, timed and spread-round launches of that run. "
        "`alg.` is the algorithmic fraction of the dtype's vector peak (157.3 TFLOP/s FP32 with "
        "packed FMA, 78.6 FP64); `exec.` the executed FLOP rate's fraction "
        "(SQ_INSTS_VALU_FLOPS counter); `busy` VALU instructions x 4 cycles over the SIMDs' "
        "cycles; `div.` VALU instructions over those of the replicated batch (lockstep ideal); "
        "`HBM` measured bytes over algorithmic bytes. The last four come from the counter "
        "records `profiles/counters_<workload>_<jobz>.json` (profile_counters.py); `CPU` is "
        "the oracle on the host's cores (bench.py `cpu_baseline`).", "",
        "| case | kernel | trace avg (us) | min | max | bench.py (us) | matrices/s | alg. | exec. "
        "| busy | div. | HBM | CPU us/matrix |",
        "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for c in order:
        r = recs[c]
        b, s = r["bench"], r["solver"]
        rf = b["roofline"]
        ex = (rf.get("executed") or {}).get("frac")
        hb = (rf["traffic"] / b["hbm"]["algorithmic_bytes_per_launch"]
              if rf.get("traffic") else None)
        cpu = (b.get("cpu_baseline") or {}).get("us_per_matrix")
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.2f | %.3g | %s | %s | %s | %s | %s | %s |" % (
            c.replace(":", " "), rf["kernel"], s["avg_us"], s["min_us"], s["max_us"],
            b["ms_per_step"] * 1e3, b["value"], fmt(rf["frac"], "%.4f"), fmt(ex, "%.4f"),
            fmt(rf.get("valu_busy"), "%.2f"), fmt(rf.get("divergence"), "%.3f"),
            fmt(hb, "%.3f"), fmt(cpu, "%.3f")))
    if order:
        out = os.path.join(ROOT, "profiles", "steqr_all_workloads_trace.md")
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", out)
    if HEADLINE in recs:
        write_headline(recs[HEADLINE])
    for mode, (fname, title, cases) in EXTRA_SETS.items():
        have = [c for c in cases if c in recs]
        if have:
            write_extra(mode, fname, title, have, recs)


def write_extra(mode: str, fname: str, title: str, cases, recs) -> None:
    """Summary of one option set, with the plain (QR, no basis) time of the
    same workload from the same directory for comparison where it exists."""
    lines = ["# %s, one MI355X" % title, "",
             "Per case, bench.py and a rocprofv3 kernel trace of the same command, from:", "",
             "    python3 profile_workloads.py --out OUT " + " ".join(cases),
             "    python3 profile_workloads.py --summarise OUT", "",
             "which runs, per case:", "",
             "    python3 bench.py --workload WL --jobz J --steps S --warmup 5 %s" % " ".join(MODES[mode]),
             "    rocprofv3 --kernel-trace --stats -d OUT -o run --output-format csv -- python3 bench.py "
             "--workload WL --jobz J --steps S --warmup 5 %s --no-cpu --no-named --no-saturation"
             % " ".join(MODES[mode]), "",
             "`alg.`: algorithmic fraction of the dtype's vector peak (157.3 TFLOP/s FP32 with packed "
             "FMA, 78.6 FP64); `exec.`, `busy`, `div.`, `HBM`: executed fraction, VALU busy, "
             "divergence and measured over algorithmic HBM bytes from the option set's counter "
             "record (profiles/counters_<workload>_<jobz>_<set>.json, where one was taken); "
             "`plain`: the default solve of the same workload (EXP step, QR, no basis) from the "
             "records summarised in steqr_all_workloads_trace.md.", "",
             "| case | kernel | trace avg (us) | bench.py (us) | matrices/s | alg. | exec. | busy "
             "| div. | HBM | plain (us) | ratio | CPU oracle us/matrix |",
             "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for c in cases:
        r = recs[c]
        b, s = r["bench"], r["solver"]
        rf = b.get("roofline") or {}
        wname, j, _ = split_case(c)
        plain = recs.get("%s:%s" % (wname, j))
        pt = plain["bench"]["ms_per_step"] * 1e3 if plain else None
        t = b["ms_per_step"] * 1e3
        cpu = (b.get("cpu_baseline") or {}).get("us_per_matrix")
        ex = (rf.get("executed") or {}).get("frac")
        hb = (rf["traffic"] / b["hbm"]["algorithmic_bytes_per_launch"]
              if rf.get("traffic") else None)
        lines.append("| %s %s | %s | %.2f | %.2f | %.3g | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            wname, j, s["name"].split("(")[0].replace("void ", ""), s["avg_us"], t, b["value"],
            fmt(rf.get("frac"), "%.4f"), fmt(ex, "%.4f"), fmt(rf.get("valu_busy"), "%.2f"),
            fmt(rf.get("divergence"), "%.3f"), fmt(hb, "%.3f"), fmt(pt, "%.2f"),
            fmt(t / pt if pt else None, "%.3f"), fmt(cpu, "%.3f")))
    out = os.path.join(ROOT, "profiles", fname)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


def write_headline(r: dict) -> None:
    b, s = r["bench"], r["solver"]
    rf = b["roofline"]
    ctr = json.load(open(os.path.join(ROOT, "profiles", "counters_c2_f32_n16_V.json")))
    raw = ctr["raw"]
    v, vr, fl = raw["valu"], raw["valu_replicated"], raw["flops"]
    clk = v["SQ_BUSY_CYCLES"] / 32.0 / v["dur_us"] / 1e3
    lines = [
        "# %s — float32, n = 16, batch 32,768" % rf["kernel"], "",
        "Workload: 32,768 symmetric tridiagonal matrices of order 16, d and e iid N(0,1) "
        "(workloads.py c2_f32_n16), eigenvalues and eigenvectors, default launch (%d lanes per "
        "problem, %d rows of Q per lane, band in registers, %d wavefronts per workgroup, %d "
        "workgroups). One MI355X." % (b["config"]["lanes_per_problem"],
                                     b["config"]["rows_per_lane"],
                                     b["config"]["waves_per_block"], b["config"]["workgroups"]),
        "", "## Kernel trace", "", "    " + r["trace_command"], "",
        "| kernel | calls | total (us) | avg (us) | min (us) | max (us) |", "|---|---:|---:|---:|---:|---:|"]
    for t in r["trace"]:
        lines.append("| %s | %d | %.1f | %.2f | %.2f | %.2f |" % (
            t["name"], t["calls"], t["total_us"], t["avg_us"], t["min_us"], t["max_us"]))
    lines += ["", "bench.py's HIP-event mean over the timed region in the same session: %.2f us "
              "per launch (`%s`; roofline.frac %.4f, executed.frac %s)." % (
                  b["ms_per_step"] * 1e3, r["bench_command"], rf["frac"],
                  fmt((rf.get("executed") or {}).get("frac"), "%.4f")), "",
              "## Counters (per dispatch, from profiles/counters_c2_f32_n16_V.json)", ""]
    lines += ["    " + c for c in ctr["commands"]]
    lines += ["", "| counter | random batch | replicated batch (lockstep ideal) |", "|---|---:|---:|"]
    for k in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU",
              "SQ_BUSY_CYCLES"):
        lines.append("| %s | %s | %s |" % (k, "{:,.0f}".format(v[k]), "{:,.0f}".format(vr[k])))
    lines.append("| dispatch duration (us) | %.1f | %.1f |" % (v["dur_us"], vr["dur_us"]))
    lines += ["", "| FP32 instruction counter (random batch) | value |", "|---|---:|"]
    for k in ("SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32",
              "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_FLOPS_FP32", "SQ_INSTS_VALU_INT32",
              "SQ_INSTS_VALU"):
        lines.append("| %s | %s |" % (k, "{:,.0f}".format(fl[k])))
    arith = (fl["SQ_INSTS_VALU_FMA_F32"] + fl["SQ_INSTS_VALU_MUL_F32"] + fl["SQ_INSTS_VALU_ADD_F32"]
             + fl["SQ_INSTS_VALU_TRANS_F32"])
    other = fl["SQ_INSTS_VALU"] - arith - fl["SQ_INSTS_VALU_INT32"]
    lines += ["", "Derived:",
              "* divergence = VALU instructions, random / replicated = %.3f the lockstep ideal "
              "(VALU + SALU: %.3f);" % (v["SQ_INSTS_VALU"] / vr["SQ_INSTS_VALU"],
                                       (v["SQ_INSTS_VALU"] + v["SQ_INSTS_SALU"])
                                       / (vr["SQ_INSTS_VALU"] + vr["SQ_INSTS_SALU"])),
              "* clock from SQ_BUSY_CYCLES: %.2f GHz;" % clk,
              "* VALU busy = VALU instructions x 4 cycles / (1,024 SIMDs x the dispatch's cycles) "
              "= %.0f%%;" % (100 * rf.get("valu_busy", 0)),
              "* instruction mix: FP32 arithmetic %.0f%%, INT32 %.0f%%, other (moves, selects, "
              "compares, lane moves) %.0f%%;" % (100 * arith / fl["SQ_INSTS_VALU"],
                                                 100 * fl["SQ_INSTS_VALU_INT32"] / fl["SQ_INSTS_VALU"],
                                                 100 * other / fl["SQ_INSTS_VALU"]),
              "* executed FP32 flops = 64 lanes x FLOPS counter = %.3g per launch; at the timed "
              "mean %.1f TFLOP/s = %.1f%% of 157.3 (packed) and %.1f%% of the 78.6 non-packed "
              "rate;" % (ctr["executed_flops_per_launch"], rf["executed"]["tflops"],
                         100 * rf["executed"]["frac"], 100 * rf["executed"]["frac_nonpacked"]),
              "* algorithmic flops (CPU oracle rotation counts, bench.py model) = %.3g per "
              "launch = %.1f TFLOP/s = %.1f%% of 157.3 (%.1f%% of 78.6)." % (
                  rf["algorithmic_flops_per_launch"], rf["achieved"], 100 * rf["frac"],
                  100 * rf["frac_nonpacked"]), "",
              "## HBM traffic", "",
              "FETCH_SIZE and WRITE_SIZE scaled by a plain device copy / fill of 256 MiB (fetch x%.4f, "
              "write x%.4f): %.4g bytes per launch against %.4g algorithmic (%.3fx)." % (
                  ctr["calibration"]["fetch_factor"], ctr["calibration"]["write_factor"],
                  ctr["hbm_bytes_per_launch"], ctr["algorithmic_bytes_per_launch"],
                  ctr["hbm_bytes_per_launch"] / ctr["algorithmic_bytes_per_launch"]), "",
              "Phase split and wavefront timeline of the same kernel: "
              "profiles/phases_c2_f32_n16_V.md."]
    out = os.path.join(ROOT, "profiles", "steqr_chunk_f32_n16_V_headline.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("cases", nargs="*", default=CASES)
    ap.add_argument("--out", default=None, help="directory for the per-case JSON files")
    ap.add_argument("--summarise", default=None, metavar="DIR",
                    help="write the profiles/ summaries from DIR's JSON files")
    ap.add_argument("--timeout", type=int, default=240, help="seconds per step")
    args = ap.parse_args()
    if args.summarise:
        summarise(args.summarise)
        return 0
    if not args.out:
        ap.error("--out is required to collect")
    os.environ.setdefault("TMPDIR", "/tmp")
    os.makedirs(args.out, exist_ok=True)
    for c in args.cases:
        print("case", c, flush=True)
        collect(c, args.out, args.timeout)
    return 0


if __name__ == "__main__":
    sys.exit(main())
