"""GPU parity at orders 65..512 (producer and consumer wavefronts with
eigenvectors, rows of Q split over lanes and, from order 256 in double and
512 in float, over workgroups; producer wavefronts alone for values only)
against the oracle on the same seeded inputs. Needs an MI355X; run with
-m gpu."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, check_basis, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [65, 66, 77, 96, 100, 127, 128])
def test_big_orders(n, dt, jobz):
    print("big case", n, dt.__name__, jobz, flush=True)
    d, e = W.random_batch(n, 203, dt, salt=500 + n)
    g = run_gpu(d, e, jobz)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [90, 128])
def test_big_edge_items(kind, dt, n):
    print("big edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    d, e = W.edge_batch(kind, n, 70, dt)
    for jobz in (True, False):
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz, threads=8)
        assert check(d, e, g, o, jobz) == [], (W.EDGE_NAMES[kind], jobz)
        if kind == W.EDGE_NAN:
            assert np.all(g[2] > 0)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_big_schemes_shift_and_basis(dt):
    n = 128
    d, e = W.random_batch(n, 150, dt, salt=510)
    for scheme, shift in ((1, 0), (0, 1), (1, 1)):
        print("big scheme/shift", dt.__name__, scheme, shift, flush=True)
        for jobz in (True, False):
            g = run_gpu(d, e, jobz, scheme=scheme, shift=shift)
            o = oracle.steqr(d, e, jobz, threads=8, scheme=scheme, shift=shift)
            assert check(d, e, g, o, jobz) == [], (scheme, shift, jobz)
    Z = W.random_basis(n, 150, dt, salt=511)
    g = run_gpu(d, e, True, Z=Z)
    o = oracle.steqr(d, e, True, threads=8, Z=Z)
    assert check_basis(d, e, Z, g, o) == []


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_big_unsorted_and_budget(dt):
    n = 100
    d, e = W.random_batch(n, 120, dt, salt=512)
    g = run_gpu(d, e, True, sort=False)
    o = oracle.steqr(d, e, True, sort=False, threads=8)
    # unsorted: compare sorted eigenvalues and the residual of the pairs
    assert check(d, e, (np.sort(g[0], 1), None, g[2]), (np.sort(o[0], 1), None, o[2]), False) == []
    import validate as V
    assert V.band_residual(d, e, g[0], g[1]).max() <= V.tol_of(dt, n)
    # a budget of one sweep per eigenvalue fails the same items (the state
    # at the failure depends on rounding, so only the status is compared)
    g = run_gpu(d, e, True, max_sweeps_per_n=1)
    o = oracle.steqr(d, e, True, max_sweeps_per_n=1, threads=8)
    assert np.array_equal(g[2] > 0, o[2] > 0)
    g = run_gpu(d, e, False, max_sweeps_per_n=-1)
    o = oracle.steqr(d, e, False, max_sweeps_per_n=0, threads=8)
    assert np.array_equal(g[2], o[2]) and np.all(g[2] > 0) and np.array_equal(g[0], d)


@pytest.mark.parametrize("dt,lanes", [(np.float32, 8), (np.float32, 16), (np.float32, 32),
                                      (np.float64, 16), (np.float64, 32)],
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_big_producer_shapes(dt, lanes):
    """Every built (producer lanes, consumers per workgroup) shape at order 128."""
    for n in (80, 128):
        print("big shape", dt.__name__, lanes, n, flush=True)
        d, e = W.random_batch(n, 150, dt, salt=520 + n)
        g = run_gpu(d, e, True, lanes=lanes)
        o = oracle.steqr(d, e, True, threads=8)
        assert check(d, e, g, o, True) == []


@pytest.mark.parametrize("dt,lanes", [(np.float32, 8), (np.float32, 16), (np.float64, 8),
                                      (np.float64, 16)],
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_big_values_shapes(dt, lanes):
    """Every built producer shape of the values-only kernel at order 128."""
    for n in (70, 128):
        print("big values shape", dt.__name__, lanes, n, flush=True)
        d, e = W.random_batch(n, 150, dt, salt=530 + n)
        g = run_gpu(d, e, False, lanes=lanes)
        o = oracle.steqr(d, e, False, threads=8)
        assert check(d, e, g, o, False) == []


# ---------------------------------------------------------------- orders 129..256
# Producer and consumer wavefronts at compiled order 256: one problem per
# producer, rows of Q split over two (float) or four (double) lanes, double
# with two workgroups sharing each problem's rows; values only with one
# problem per producer wavefront (two or four selectable).

@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [129, 130, 191, 200, 255, 256])
def test_huge_orders(n, dt, jobz):
    print("huge case", n, dt.__name__, jobz, flush=True)
    d, e = W.random_batch(n, 61, dt, salt=600 + n)
    g = run_gpu(d, e, jobz)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_huge_edge_items(kind, dt):
    n = 256
    print("huge edge", W.EDGE_NAMES[kind], dt.__name__, flush=True)
    d, e = W.edge_batch(kind, n, 30, dt)
    for jobz in (True, False):
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz, threads=8)
        assert check(d, e, g, o, jobz) == [], (W.EDGE_NAMES[kind], jobz)
        if kind == W.EDGE_NAN:
            assert np.all(g[2] > 0)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_huge_schemes_shift_basis_and_lanes(dt):
    n = 240
    d, e = W.random_batch(n, 40, dt, salt=610)
    for scheme, shift in ((1, 0), (0, 1)):
        print("huge scheme/shift", dt.__name__, scheme, shift, flush=True)
        for jobz in (True, False):
            g = run_gpu(d, e, jobz, scheme=scheme, shift=shift)
            o = oracle.steqr(d, e, jobz, threads=8, scheme=scheme, shift=shift)
            assert check(d, e, g, o, jobz) == [], (scheme, shift, jobz)
    Z = W.random_basis(n, 40, dt, salt=611)
    g = run_gpu(d, e, True, Z=Z)
    o = oracle.steqr(d, e, True, threads=8, Z=Z)
    assert check_basis(d, e, Z, g, o) == []
    # values only with four problems per producer wavefront (16 lanes each)
    g = run_gpu(d, e, False, lanes=16)
    o = oracle.steqr(d, e, False, threads=8)
    assert check(d, e, g, o, False) == []
    # unsorted output and a sweep budget of zero
    g = run_gpu(d, e, True, sort=False)
    o = oracle.steqr(d, e, True, sort=False, threads=8)
    assert check(d, e, (np.sort(g[0], 1), None, g[2]), (np.sort(o[0], 1), None, o[2]), False) == []
    g = run_gpu(d, e, True, max_sweeps_per_n=-1)
    assert np.all(g[2] > 0)


# ---------------------------------------------------------------- orders 257..512
# Compiled order 512: one problem per producer; rows of Q split over eight
# (float) or sixteen (double) lanes, and over eight (float) or sixteen
# (double) workgroups per problem, each with its own producer.

@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [257, 300, 383, 511, 512])
def test_n512_orders(n, dt, jobz):
    print("n512 case", n, dt.__name__, jobz, flush=True)
    d, e = W.random_batch(n, 13, dt, salt=700 + n)
    g = run_gpu(d, e, jobz)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_n512_edge_items(kind, dt):
    n = 512
    print("n512 edge", W.EDGE_NAMES[kind], dt.__name__, flush=True)
    d, e = W.edge_batch(kind, n, 6, dt)
    for jobz in (True, False):
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz, threads=8)
        assert check(d, e, g, o, jobz) == [], (W.EDGE_NAMES[kind], jobz)
        if kind == W.EDGE_NAN:
            assert np.all(g[2] > 0)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_n512_schemes_shift_basis_and_lanes(dt):
    n = 450
    d, e = W.random_batch(n, 6, dt, salt=710)
    for scheme, shift in ((1, 0), (0, 1)):
        print("n512 scheme/shift", dt.__name__, scheme, shift, flush=True)
        for jobz in (True, False):
            g = run_gpu(d, e, jobz, scheme=scheme, shift=shift)
            o = oracle.steqr(d, e, jobz, threads=8, scheme=scheme, shift=shift)
            assert check(d, e, g, o, jobz) == [], (scheme, shift, jobz)
    Z = W.random_basis(n, 6, dt, salt=711)
    g = run_gpu(d, e, True, Z=Z)
    o = oracle.steqr(d, e, True, threads=8, Z=Z)
    assert check_basis(d, e, Z, g, o) == []
    g = run_gpu(d, e, True, sort=False)
    o = oracle.steqr(d, e, True, sort=False, threads=8)
    assert check(d, e, (np.sort(g[0], 1), None, g[2]), (np.sort(o[0], 1), None, o[2]), False) == []
    g = run_gpu(d, e, True, max_sweeps_per_n=-1)
    assert np.all(g[2] > 0)


@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_orders_65_to_512_sampled(dt, jobz):
    """Every 17th order from 65 to 512 (each compiled order with a range of
    padding, ragged row slices of Q and, from 257, problems shared by several
    workgroups), a few items each."""
    for n in range(65, 513, 17):
        print("order sweep", dt.__name__, jobz, n, flush=True)
        d, e = W.random_batch(n, 5, dt, salt=900 + n)
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz, threads=8)
        assert check(d, e, g, o, jobz) == [], "n=%d" % n
