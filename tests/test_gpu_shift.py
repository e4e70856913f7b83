"""GPU parity of the closed-form lambda+- shift (steqr_params.shift =
STEQR_SHIFT_CLOSED) against the oracle with the same shift, alone and with
the PG update scheme. Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import validate as V
import workloads as W
from parity import check, run_gpu

pytestmark = pytest.mark.gpu

CLOSED = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


SMALL = 1000 + 13


@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
@pytest.mark.parametrize("wname", W.SMALL_BATCH_WORKLOADS)
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_closed_shift_workload_small_batch(wname, jobz, scheme):
    w = W.WORKLOADS[wname]
    print("closed-shift case %s jobz=%s scheme=%d" % (w.name, jobz, scheme), flush=True)
    d, e = W.make_batch(w, SMALL)
    g = run_gpu(d, e, jobz, scheme=scheme, shift=CLOSED)
    o = oracle.steqr(d, e, jobz, threads=8, scheme=scheme, shift=CLOSED)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [3, 16, 32, 64])
def test_closed_shift_edge_items(kind, dt, n):
    d, e = W.edge_batch(kind, n, 130, dt)
    print("closed-shift edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    g = run_gpu(d, e, True, shift=CLOSED)
    o = oracle.steqr(d, e, True, shift=CLOSED)
    assert check(d, e, g, o, True) == [], W.EDGE_NAMES[kind]
    if kind == W.EDGE_NAN:
        assert np.all(g[2] > 0)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_closed_shift_every_order(dt):
    for n in range(1, 65, 3):
        d, e = W.random_batch(n, 67, dt, salt=200 + n)
        print("closed-shift order", n, flush=True)
        g = run_gpu(d, e, True, shift=CLOSED)
        o = oracle.steqr(d, e, True, shift=CLOSED)
        assert check(d, e, g, o, True) == [], "n=%d" % n


def test_shifts_agree_on_gpu():
    w = W.WORKLOADS["c2_f32_n16"]
    d, e = W.make_batch(w, 4096)
    a = run_gpu(d, e, False)
    b = run_gpu(d, e, False, shift=CLOSED)
    assert not a[2].any() and not b[2].any()
    assert V.sorted_err(b[0], a[0].astype(np.float64), d, e).max() <= V.tol_of(d.dtype, w.n)
