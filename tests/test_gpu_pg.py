"""GPU parity of the PG (Parlett-Gray) form of the chase step
(steqr_params.update_scheme = STEQR_PG) against the oracle's PG sweeps, on
the same seeded inputs and to the same bar as the default EXP form. Needs an
MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import validate as V
import workloads as W
from parity import check, run_gpu

pytestmark = pytest.mark.gpu

PG = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


SMALL = 1000 + 13


@pytest.mark.parametrize("wname", W.SMALL_BATCH_WORKLOADS)
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_pg_workload_small_batch(wname, jobz):
    w = W.WORKLOADS[wname]
    print("pg case %s jobz=%s" % (w.name, jobz), flush=True)
    d, e = W.make_batch(w, SMALL)
    g = run_gpu(d, e, jobz, scheme=PG)
    o = oracle.steqr(d, e, jobz, threads=8, scheme=PG)
    assert check(d, e, g, o, jobz) == []


def test_pg_headline_full_size():
    """The full float n=16 eigenvector batch in the default launch shape:
    a spread sample against the oracle, residual and orthogonality on all."""
    w = W.WORKLOADS["c2_f32_n16"]
    d, e = W.make_batch(w)
    g = run_gpu(d, e, True, scheme=PG)
    nb = w.batch
    items = np.unique(np.concatenate([np.linspace(0, nb - 1, 384).astype(int),
                                      np.arange(nb - 40, nb)]))
    o = oracle.steqr(d[items], e[items], True, threads=8, scheme=PG)
    assert check(d, e, g, o, True, items=items) == []
    lam, Q, info = g
    assert not info.any()
    tol = V.tol_of(d.dtype, w.n)
    assert V.band_residual(d, e, lam, Q).max() <= tol
    assert V.orthogonality(Q).max() <= tol


PG_LANES = [
    # dtype, n, jobz, lanes, band
    (np.float32, 4, True, 4, 1), (np.float32, 8, True, 2, 1), (np.float32, 16, True, 4, 1),
    (np.float32, 16, True, 16, 1), (np.float32, 16, True, 4, 2), (np.float32, 32, True, 8, 2),
    (np.float32, 32, True, 32, 1), (np.float32, 32, False, 2, 1), (np.float32, 16, False, 1, 1),
    (np.float64, 12, True, 4, 2), (np.float64, 16, True, 8, 1), (np.float64, 32, True, 16, 2),
    (np.float64, 32, False, 1, 1), (np.float64, 8, True, 4, 1),
    (np.float32, 64, True, 64, 2), (np.float64, 64, False, 64, 2),
    (np.float64, 64, True, 4, 3), (np.float32, 40, True, 16, 3), (np.float64, 50, True, 16, 3),
]


@pytest.mark.parametrize("dt,n,jobz,lanes,band", PG_LANES,
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_pg_lanes_and_band_variants(dt, n, jobz, lanes, band):
    d, e = W.random_batch(n, 777, dt, salt=23)
    print("pg lanes case", dt.__name__, n, jobz, lanes, band, flush=True)
    g = run_gpu(d, e, jobz, lanes=lanes, band=band, scheme=PG)
    o = oracle.steqr(d, e, jobz, threads=8, scheme=PG)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [3, 16, 32, 64])
def test_pg_edge_items(kind, dt, n):
    d, e = W.edge_batch(kind, n, 130, dt)
    print("pg edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    for jobz in (True, False):
        g = run_gpu(d, e, jobz, scheme=PG)
        o = oracle.steqr(d, e, jobz, scheme=PG)
        assert check(d, e, g, o, jobz) == [], (W.EDGE_NAMES[kind], jobz)
    if kind == W.EDGE_ZERO:
        assert np.all(g[0] == 0)
    if kind == W.EDGE_NAN:
        assert np.all(g[2] > 0)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_pg_every_order_up_to_64(dt):
    for n in range(1, 65):
        d, e = W.random_batch(n, 67, dt, salt=100 + n)
        print("pg order", n, flush=True)
        g = run_gpu(d, e, True, scheme=PG)
        o = oracle.steqr(d, e, True, scheme=PG)
        assert check(d, e, g, o, True) == [], "n=%d" % n


def test_pg_nan_confined_to_block():
    n = 12
    d, e = W.random_batch(n, 8, np.float64, salt=3)
    e[:, 5] = 0.0
    d[:, 8] = np.nan
    g = run_gpu(d, e, True, scheme=PG)
    o = oracle.steqr(d, e, True, scheme=PG)
    assert check(d, e, g, o, True) == []
    assert np.all(g[2] == 5)
    assert np.all(np.isfinite(g[0][:, :6])) and np.all(np.isnan(g[0][:, 6:]))


def test_pg_and_exp_agree_on_gpu():
    """Both forms of the step give the same eigenvalues to the tolerance."""
    w = W.WORKLOADS["c4_f64_n32"]
    d, e = W.make_batch(w, 2048)
    a = run_gpu(d, e, False)
    b = run_gpu(d, e, False, scheme=PG)
    assert np.array_equal(a[2] > 0, b[2] > 0)
    ok = a[2] == 0
    assert V.sorted_err(b[0][ok], a[0][ok].astype(np.float64), d[ok], e[ok]).max() <= \
        V.tol_of(d.dtype, w.n)
