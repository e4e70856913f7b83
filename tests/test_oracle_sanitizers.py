"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only) runs the quick pins with no sanitizer report: no
out-of-bounds access, use of freed memory, signed overflow or other
undefined behaviour on the paths the pins exercise (every public routine,
both precisions, both update schemes and shifts, back-transformation, the
dense front end and bisection)."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name: str) -> str:
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_pins_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(out_dir=str(tmp_path), extra_flags=(
        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
        "-fno-omit-frame-pointer", "-g"))
    script = textwrap.dedent("""
        import sys
        sys.path[:0] = [%r, %r]
        import oracle, oracle_pins as P
        fails = P.run_all(oracle, libpath=%r, quick=True)
        print("FAILS", len(fails))
        for f in fails[:10]:
            print(f)
        sys.exit(1 if fails else 0)
    """ % (ROOT, HERE, lib))
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                       timeout=900)
    report = r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, r.stdout[-2000:] + report
