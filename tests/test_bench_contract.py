"""bench.py's output contract: one JSON line with the metric, the whole-job
value, the timing fields, the workload config, the roofline of the dominant
kernel (with the HBM traffic from the counter record) and the CPU oracle
baseline; more than one GPU is refused with a message. The GPU run is a
child process (a few launches of the headline workload)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench contract run", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "10",
                        "--warmup", "2"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    b = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                 ("steps", int), ("warmup", int), ("ms_per_step", float),
                 ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                 ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(b[k], t), k
    assert (b["n_gpus"], b["steps"], b["warmup"]) == (1, 10, 2)
    assert b["higher_is_better"] is True and b["dtype"] == "f32" and b["vs_baseline"] is None
    assert b["config"]["workload"] == "c2_f32_n16" and b["config"]["batch"] == 32768
    assert abs(b["value"] - b["config"]["batch"] / (b["ms_per_step"] * 1e-3)) <= 1e-6 * b["value"]
    rf = b["roofline"]
    assert rf["bound"] == "alu" and rf["unit"] == "TFLOP/s" and rf["peak"] == 157.3
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert 0.0 < rf["frac"] < 1.0
    assert rf["traffic"] is not None and rf["traffic"] > 0
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["unit"] == b["unit"] and isinstance(cb["sample"], str)
