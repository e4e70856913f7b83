"""GPU parity of the fused small-n dense eigensolver (syev_batched_ex:
Householder reduction, tridiagonal solve and back-transformation in one
kernel) against the oracle's syev on the same seeded matrices: status,
eigenvalues within 16 n eps ||A||, dense residual and orthogonality. Needs
an MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, check_dense, run_gpu, run_gpu_syev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


def _vectors_ok(dt, n: int) -> bool:
    """Double precision with eigenvectors is built up to SYEV_MAX_N_F64_V
    (order 32, the last with the band in LDS)."""
    import symmetric_tridiagonal_eigensolver_amd as st
    return dt != np.float64 or n <= st.SYEV_MAX_N_F64_V


# every instantiated (dtype, compiled order, lanes) at full and ragged orders
CASES = [
    (np.float32, 4, 4, True), (np.float32, 3, 4, True), (np.float32, 8, 2, True),
    (np.float32, 7, 4, True), (np.float32, 16, 4, True), (np.float32, 13, 8, True),
    (np.float32, 32, 16, True), (np.float32, 27, 16, True),
    (np.float32, 4, 4, False), (np.float32, 8, 2, False), (np.float32, 16, 4, False),
    (np.float32, 11, 4, False), (np.float32, 32, 16, False),
    (np.float64, 4, 4, True), (np.float64, 8, 4, True), (np.float64, 16, 8, True),
    (np.float64, 12, 8, True), (np.float64, 32, 32, True), (np.float64, 27, 32, True),
    (np.float64, 17, 32, True),
    (np.float64, 4, 4, False), (np.float64, 8, 4, False), (np.float64, 16, 8, False),
    (np.float64, 32, 32, False), (np.float64, 21, 32, False),
    (np.float32, 8, 1, False), (np.float32, 16, 2, False), (np.float32, 14, 2, False),
    (np.float32, 32, 8, False), (np.float32, 25, 8, False),
    (np.float64, 8, 2, False), (np.float64, 16, 4, False), (np.float64, 10, 4, False),
]


@pytest.mark.parametrize("dt,n,lanes,jobz", CASES,
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_syev_variants(dt, n, lanes, jobz):
    print("syev case", dt.__name__, n, lanes, jobz, flush=True)
    A = W.random_symmetric(n, 777, dt, salt=61)
    g = run_gpu_syev(A, jobz, lanes=lanes)
    o = oracle.syev(A, jobz, threads=8)
    assert check_dense(A, g, o, jobz) == []


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_syev_every_order(dt):
    for n in range(1, 33):
        print("syev order", dt.__name__, n, flush=True)
        A = W.random_symmetric(n, 67, dt, salt=300 + n)
        for jobz in ((True, False) if _vectors_ok(dt, n) else (False,)):
            g = run_gpu_syev(A, jobz)
            o = oracle.syev(A, jobz)
            assert check_dense(A, g, o, jobz) == [], (n, jobz)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [1, 2, 5, 16, 32])
def test_syev_special_matrices(dt, n):
    """Zero, diagonal, tridiagonal, scaled (1e+-18 / 1e+-150) and NaN items in
    one batch; the upper triangle is never read."""
    print("syev special", dt.__name__, n, flush=True)
    if not _vectors_ok(dt, n):
        pytest.skip("double with eigenvectors is built up to order 16")
    A = W.random_symmetric(n, 60, dt, salt=62)
    A[0:5] = 0
    idx = np.arange(n)
    D = np.zeros((5, n, n), dtype=dt)
    D[:, idx, idx] = W.random_batch(n, 5, dt, salt=63)[0]
    A[5:10] = D
    td, te = W.random_batch(n, 5, dt, salt=64)
    A[10:15] = W.dense_from_bands(td, te)
    big = 1e18 if dt == np.float32 else 1e150
    A[15:20] *= dt(big)
    A[20:25] *= dt(1 / big)
    A[25, n - 1, 0] = np.nan
    A[26, 0, 0] = np.nan
    g = run_gpu_syev(A, True)
    o = oracle.syev(A, True)
    assert check_dense(A, g, o, True) == []
    # only the lower triangle is read: poison the strict upper triangle
    P = A.copy()
    iu = np.triu_indices(n, 1)
    P[:, iu[0], iu[1]] = dt(3.25)
    h = run_gpu_syev(P, True)
    assert np.array_equal(h[0], g[0], equal_nan=True) and np.array_equal(h[2], g[2])
    assert np.array_equal(h[1], g[1], equal_nan=True)
    # a tridiagonal A is already reduced: the same eigenvalues as the
    # tridiagonal solver on its bands
    s = run_gpu(td, te, True)
    assert check(td, te, (g[0][10:15], g[1][10:15], g[2][10:15]), s, True) == []


def test_syev_zero_budget_and_no_sort():
    A = W.random_symmetric(16, 100, np.float32, salt=65)
    g = run_gpu_syev(A, True, max_sweeps_per_n=-1)
    o = oracle.syev(A, True, max_sweeps_per_n=0)
    assert np.array_equal(g[2], o[2]) and np.all(g[2] > 0)
    g = run_gpu_syev(A, True, sort=False)
    o = oracle.syev(A, True, sort=False)
    assert check_dense(A, g, o, True, sort=False) == []


@pytest.mark.parametrize("shift", [0, 1], ids=["lapack_shift", "closed_shift"])
@pytest.mark.parametrize("dt,n", [(np.float32, 16), (np.float32, 32), (np.float64, 16),
                                  (np.float64, 32)])
def test_syev_workload_batches(dt, n, shift):
    print("syev workload", dt.__name__, n, shift, flush=True)
    jobz = _vectors_ok(dt, n)
    A = W.random_symmetric(n, 4099, dt, salt=66)
    g = run_gpu_syev(A, jobz, shift=shift)
    o = oracle.syev(A, jobz, threads=8, shift=shift)
    assert check_dense(A, g, o, jobz) == []


@pytest.mark.parametrize("n", [32, 21])
@pytest.mark.parametrize("band", [1, 2])
def test_syev_double_order32_band_storage(n, band):
    """Double at order 32 values only: the band in registers and in LDS (the
    default) both agree with the oracle."""
    print("syev f64 values only, band", band, "n", n, flush=True)
    A = W.random_symmetric(n, 999, np.float64, salt=67)
    g = run_gpu_syev(A, False, band=band)
    o = oracle.syev(A, False, threads=8)
    assert check_dense(A, g, o, False) == []


def test_syev_double_vectors_limit():
    """Double precision with eigenvectors above order 32 is rejected (-4)
    before any launch; at order 32 double runs with the band in LDS by
    default."""
    import symmetric_tridiagonal_eigensolver_amd as st
    assert st.lib().syev_batched(8, 8, 8, 33, 10, st.STEQR_V, st.STEQR_F64, None) == -4
    q = st.syev_query(32, 10, st.STEQR_N, st.STEQR_F64)
    assert (q["lanes_per_problem"], q["band_storage"]) == (32, 2)
    q = st.syev_query(17, 10, st.STEQR_V, st.STEQR_F64)
    assert (q["lanes_per_problem"], q["band_storage"]) == (32, 2)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [2, 5, 16, 32])
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_syev_infinite_entries(dt, n, jobz):
    """Items with +-inf in the lower triangle among ordinary ones: status
    and NaN positions as the oracle's."""
    print("syev infinite", dt.__name__, n, jobz, flush=True)
    if jobz and not _vectors_ok(dt, n):
        pytest.skip("double with eigenvectors is built up to order 16")
    A = W.random_symmetric(n, 40, dt, salt=67)
    g = np.random.default_rng(n + 3)
    for b in range(0, 40, 4):
        i = int(g.integers(0, n))
        j = int(g.integers(0, i + 1))
        v = np.inf if g.random() < 0.5 else -np.inf
        A[b, i, j] = v
        A[b, j, i] = v
    gpu = run_gpu_syev(A, jobz)
    o = oracle.syev(A, jobz)
    assert check_dense(A, gpu, o, jobz) == []
