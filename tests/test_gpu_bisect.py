"""GPU parity of the values-only bisection (steqr_params.method =
STEQR_METHOD_BISECT) against the oracle's bisection on the same seeded
inputs: status, eigenvalues within 16 n eps ||T||, ascending order; plus
the exact power-of-two scaling the method has by construction, and
agreement with the QR solve. Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import validate as V
import workloads as W
from parity import check, run_gpu

pytestmark = pytest.mark.gpu

BISECT = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


def run_bisect(d, e, **kw):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    dev = torch.device("cuda:0")
    td = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    te = torch.from_numpy(np.ascontiguousarray(e)).to(dev)
    lam, _, info = st.solve(td, te, False, info=True, method=BISECT, **kw)
    torch.cuda.synchronize()
    return lam.cpu().numpy(), None, info.cpu().numpy()


def oracle_bisect(d, e):
    lam, info = oracle.stebz(d, e, threads=8)
    return lam, None, info


BISECT_WORKLOADS = list(W.WORKLOADS)


@pytest.mark.parametrize("wname", BISECT_WORKLOADS)
def test_bisect_workload_small_batch(wname):
    w = W.WORKLOADS[wname]
    print("bisect case", wname, flush=True)
    d, e = W.make_batch(w, 1000 + 13)
    g = run_bisect(d, e)
    o = oracle_bisect(d, e)
    assert check(d, e, g, o, False) == []


@pytest.mark.parametrize("wname", ["c2_f32_n16", "c4_f32_n32", "c4_f64_n32", "c5_f64_n64",
                                   "w_f32_n128", "w_f64_n128", "w_f32_n256", "w_f64_n512"])
def test_bisect_full_batch_sampled(wname):
    """The full batch in the benchmark's launch; the oracle on every 64th item."""
    w = W.WORKLOADS[wname]
    print("bisect full", wname, flush=True)
    d, e = W.make_batch(w)
    g = run_bisect(d, e)
    items = np.arange(0, d.shape[0], 64)
    o = oracle_bisect(d[items], e[items])
    assert check(d, e, g, o, False, items=items) == []


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_bisect_every_order(dt):
    for n in list(range(1, 65)) + [65, 70, 96, 127, 128, 129, 200, 256, 257, 300, 511, 512]:
        print("bisect order", dt.__name__, n, flush=True)
        d, e = W.random_batch(n, 67, dt, salt=400 + n)
        g = run_bisect(d, e)
        o = oracle_bisect(d, e)
        assert check(d, e, g, o, False) == [], "n=%d" % n


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [1, 2, 3, 16, 32, 64, 100, 128, 256, 512])
def test_bisect_edge_items(kind, dt, n):
    print("bisect edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    d, e = W.edge_batch(kind, n, 130, dt)
    g = run_bisect(d, e)
    o = oracle_bisect(d, e)
    assert check(d, e, g, o, False) == [], W.EDGE_NAMES[kind]
    if kind == W.EDGE_NAN:
        assert np.all(g[2] == n) and np.all(np.isnan(g[0]))


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [5, 16, 64, 128, 256, 512])
def test_bisect_power_of_two_scaling_is_exact(dt, n):
    d, e = W.random_batch(n, 200, dt, salt=76)
    base = run_bisect(d, e)[0]
    for j in (-50, 9, 40):
        f = dt(2.0 ** j)
        assert np.array_equal(run_bisect(d * f, e * f)[0], base * f), j


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_bisect_agrees_with_qr_and_closed_forms(dt):
    for n in (4, 16, 33, 64, 128):
        d, e = W.random_batch(n, 500, dt, salt=77)
        g = run_bisect(d, e)
        q = run_gpu(d, e, False)
        assert not g[2].any() and not q[2].any()
        assert V.sorted_err(g[0], q[0].astype(np.float64), d, e).max() <= V.tol_of(dt, n)
        # Kac-Sylvester-Clement: eigenvalues -(n-1), -(n-3), ..., n-1
        k = np.arange(1, n)
        ce = np.sqrt(k * (n - k)).reshape(1, -1).astype(dt)
        cl = run_bisect(np.zeros((1, n), dtype=dt), ce)[0][0]
        ref = np.arange(-(n - 1), n, 2, dtype=np.float64)
        assert np.abs(cl - ref).max() <= V.tol_of(dt, n) * (2 * ce.max())


@pytest.mark.parametrize("dt,n,lanes", [
    (np.float32, 512, 128), (np.float32, 512, 256), (np.float64, 512, 128),
    (np.float64, 512, 256), (np.float64, 300, 128), (np.float32, 257, 256),
    (np.float32, 256, 128), (np.float64, 256, 256), (np.float32, 200, 256),
    (np.float64, 129, 128), (np.float32, 128, 128), (np.float64, 100, 128),
    (np.float32, 65, 128)])
def test_bisect_several_wavefronts_per_problem(dt, n, lanes):
    """A problem's indices spread over 2 or 4 wavefronts of a workgroup:
    the oracle's eigenvalues and status on a ragged batch with every edge
    kind, and the same bits as one wavefront per problem."""
    print("bisect wavefronts case", dt.__name__, n, lanes, flush=True)
    nb = 37
    d, e = W.random_batch(n, nb, dt, salt=31)
    for b in range(4, nb, 7):
        de, ee = W.edge_batch((b // 7) % 5, n, 1, dt, salt=b)
        d[b], e[b] = de[0], ee[0]
    g = run_bisect(d, e, lanes_per_problem=lanes)
    o = oracle_bisect(d, e)
    assert check(d, e, g, o, False) == []
    g1 = run_bisect(d, e, lanes_per_problem=64)
    assert np.array_equal(g[0].view(np.uint8), g1[0].view(np.uint8))
    assert np.array_equal(g[2], g1[2])


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [2, 4, 16, 64, 128, 256, 512])
def test_bisect_infinite_entries(n, dt):
    """Items with +-inf in d or e: the same status and NaN positions as the
    oracle's bisection."""
    print("bisect infinite entries", n, dt.__name__, flush=True)
    nb = 40 if n <= 64 else 12
    d, e = W.random_batch(n, nb, dt, salt=52)
    g = np.random.default_rng(n + 7)
    for b in range(0, nb, 3):
        if n > 1 and g.random() < 0.5:
            e[b, int(g.integers(0, n - 1))] = np.inf if g.random() < 0.5 else -np.inf
        else:
            d[b, int(g.integers(0, n))] = np.inf if g.random() < 0.5 else -np.inf
    assert check(d, e, run_bisect(d, e), oracle_bisect(d, e), False) == []
