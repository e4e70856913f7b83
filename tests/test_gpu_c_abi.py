"""The C ABI from a plain C program (tests/c/steqr_c_check.c, built by
__graft_entry__.build()): device memory from the HIP runtime, the 9-argument
steqr_batched and steqr_batched_ex, results checked against closed forms
(discrete Laplacians at orders 12, 37 and 300), bit-identity of the two
entry points and the argument errors. Needs an MI355X; run with -m gpu."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "steqr_c_check")


def test_c_caller():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "%s is not built (run __graft_entry__.build())" % BIN
    print("C caller", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all ok" in r.stdout
