"""Host checks of the measurement records under profiles/ and of the
profiling build: every per-launch counter record was taken on the kernel
instantiation the library's default plan runs for its workload, on the
current kernel code (bench.py reports HBM traffic and executed-instruction
figures only from such a record), and the phase-timer statements leave the
kernel code hash unchanged (they expand to nothing in the library)."""
import glob
import json
import os

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def st():
    import symmetric_tridiagonal_eigensolver_amd as st
    return st


def _records():
    return sorted(glob.glob(os.path.join(ROOT, "profiles", "counters_*.json")))


def test_every_workload_has_a_counter_record():
    have = {os.path.basename(p) for p in _records()}
    for name in W.WORKLOADS:
        for j in ("V", "N"):
            if name == "c1_f32_n4" and j == "N":
                continue  # the smallest case is timed with vectors only
            if name.startswith("c3_") and j == "N":
                continue
            assert "counters_%s_%s.json" % (name, j) in have, (name, j)


@pytest.mark.parametrize("path", _records(), ids=os.path.basename)
def test_counter_record_is_current(st, path):
    r = json.load(open(path))
    w = W.WORKLOADS[r["workload"]]
    jobz = r["jobz"] == "V"
    mode = r.get("mode", "")
    scheme, method = int(mode == "pg"), int(mode == "bisect")
    plan = st.steqr_query(w.n, w.batch, int(jobz), st.STEQR_F32 if w.dtype == "f32" else st.STEQR_F64,
                          st.make_params(update_scheme=scheme, method=method))
    fam = bench.kernel_family(plan, jobz, method)
    kname = bench.kernel_label(plan, jobz, w.dtype, fam, scheme)
    suffix = bench.record_suffix(mode == "bt", scheme, method)
    assert os.path.basename(path) == "counters_%s_%s%s.json" % (r["workload"], r["jobz"], suffix)
    assert r["kernel"] == kname
    assert r["kernel_source_hash"] == bench.kernel_source_hash(fam)
    assert bench.counters_from_profiles(r["workload"], jobz, fam, kname, suffix) is not None
    # the HBM bytes are at least the algorithmic bytes (the calibrated
    # counters cannot read less than the data that must move)
    assert r["hbm_bytes_per_launch"] >= 0.95 * r["algorithmic_bytes_per_launch"]


def test_phase_statements_do_not_change_the_hash(tmp_path, monkeypatch):
    cs = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd", "csrc")
    src = open(os.path.join(cs, "steqr_chunk.hpp")).read()
    assert "STEQR_PHASE_MARK(" in src
    stripped = bench.PHASE_TIMER_STMT.sub("", bench.strip_comments(src))
    assert "STEQR_PHASE" not in stripped and "steqr_phase.hpp" not in stripped
    # the same text with the statements removed by hand hashes the same
    import re
    plain = re.sub(r'#include "steqr_phase\.hpp"\n|[ \t]*STEQR_PHASE_[A-Z]+(\([^()]*\))?;[^\n]*\n',
                   "", src)
    assert bench.strip_comments(plain) == stripped


def test_phase_timers_are_off_in_the_library_sources():
    cs = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd", "csrc")
    for f in glob.glob(os.path.join(cs, "*.hip")):
        assert "STEQR_PHASE_TIMERS" not in open(f).read(), f
    probe = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd", "probes",
                         "steqr_phase_probe.hip")
    assert "#define STEQR_PHASE_TIMERS 1" in open(probe).read()
