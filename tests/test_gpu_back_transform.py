"""GPU parity of back-transformation (steqr_params.back_transform = 1): Q
holds a basis Z on entry and receives Z times the rotations [steqr algorithm
page, eigenvector paragraph]. Against the oracle with the same basis:
status and eigenvalues as in the plain parity tests, and the columns of Q
are orthonormal eigenvectors of A = Z T Z^T within 16 n eps. The GPU
result for a general (non-orthogonal) Z must also equal the matmul of Z
with the GPU's own plain result (the same rotations), and Z = I must
reproduce the plain solve bit for bit. Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import validate as V
import workloads as W
from parity import check, check_basis, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


# dtype, n, lanes, band: every kernel family with eigenvectors, full and
# ragged orders (n below the compiled order)
KERNEL_CASES = [
    (np.float32, 4, 4, 1), (np.float32, 8, 2, 1), (np.float32, 16, 4, 1), (np.float32, 13, 4, 1),
    (np.float32, 16, 16, 1), (np.float32, 32, 16, 1), (np.float32, 3, 1, 1),
    (np.float64, 8, 4, 1), (np.float64, 16, 8, 1), (np.float64, 16, 16, 1),
    (np.float32, 16, 4, 2), (np.float32, 32, 8, 2), (np.float32, 27, 8, 2),
    (np.float64, 16, 4, 2), (np.float64, 32, 16, 2), (np.float64, 12, 4, 2),
    (np.float32, 64, 64, 2), (np.float32, 45, 64, 2),
    (np.float32, 64, 16, 3), (np.float64, 64, 4, 3), (np.float64, 33, 16, 3),
    (np.float32, 50, 16, 3),
]


@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
@pytest.mark.parametrize("dt,n,lanes,band", KERNEL_CASES,
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_back_transform_kernels(dt, n, lanes, band, scheme):
    print("back-transform case", dt.__name__, n, lanes, band, scheme, flush=True)
    batch = 333
    d, e = W.random_batch(n, batch, dt, salt=41)
    Z = W.random_basis(n, batch, dt, salt=42)
    g = run_gpu(d, e, True, lanes=lanes, band=band, scheme=scheme, Z=Z)
    o = oracle.steqr(d, e, True, threads=8, scheme=scheme, Z=Z)
    assert check_basis(d, e, Z, g, o) == []
    # the same rotations as the plain solve: eigenvalues and status bit-equal,
    # Q equal to Z times the plain Q up to the rounding of the products
    p = run_gpu(d, e, True, lanes=lanes, band=band, scheme=scheme)
    assert np.array_equal(g[0], p[0]) and np.array_equal(g[2], p[2])
    G = W.random_basis(n, batch, dt, salt=43, orthogonal=False)
    h = run_gpu(d, e, True, lanes=lanes, band=band, scheme=scheme, Z=G)
    ref = np.matmul(G.astype(np.float64), p[1].astype(np.float64))
    rowerr = np.sqrt(((h[1].astype(np.float64) - ref) ** 2).sum(-1))
    rown = np.sqrt((G.astype(np.float64) ** 2).sum(-1))
    tol = V.tol_of(dt, n)
    assert np.all(rowerr <= tol * rown), (rowerr / rown).max()
    ident = np.ascontiguousarray(np.broadcast_to(np.eye(n, dtype=dt), (batch, n, n)))
    i = run_gpu(d, e, True, lanes=lanes, band=band, scheme=scheme, Z=ident)
    assert np.array_equal(i[1], p[1]) and np.array_equal(i[0], p[0])


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [1, 2, 16, 32, 64])
def test_back_transform_edge_items(kind, dt, n):
    print("back-transform edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    d, e = W.edge_batch(kind, n, 130, dt)
    Z = W.random_basis(n, 130, dt, salt=44)
    g = run_gpu(d, e, True, Z=Z)
    o = oracle.steqr(d, e, True, Z=Z)
    if n == 1:
        # nothing to iterate: lambda = d (NaN included, status 0) and Q = Z
        assert np.array_equal(g[0], o[0], equal_nan=True) and np.array_equal(g[2], o[2])
        assert np.array_equal(g[1], Z) and np.array_equal(o[1], Z)
    else:
        assert check_basis(d, e, Z, g, o) == [], W.EDGE_NAMES[kind]


def test_back_transform_failed_items_keep_the_basis():
    """A zero sweep budget stops unreduced blocks before any rotation: the
    failed items return Z unchanged, as the oracle does."""
    for dt, n in ((np.float32, 16), (np.float64, 32), (np.float64, 64)):
        print("back-transform budget 0", dt.__name__, n, flush=True)
        d, e = W.random_batch(n, 200, dt, salt=45)
        G = W.random_basis(n, 200, dt, salt=46, orthogonal=False)
        g = run_gpu(d, e, True, max_sweeps_per_n=-1, Z=G)
        o = oracle.steqr(d, e, True, max_sweeps_per_n=0, Z=G)
        assert np.array_equal(g[2], o[2]) and np.all(g[2] > 0)
        assert np.array_equal(g[1], G) and np.array_equal(o[1], G)


@pytest.mark.parametrize("wname", ["c2_f32_n16", "c4_f64_n32", "c5_f64_n64"])
def test_back_transform_workloads(wname):
    w = W.WORKLOADS[wname]
    print("back-transform workload", wname, flush=True)
    d, e = W.make_batch(w, 1000 + 13)
    Z = W.random_basis(w.n, d.shape[0], d.dtype, salt=47)
    g = run_gpu(d, e, True, Z=Z)
    o = oracle.steqr(d, e, True, threads=8, Z=Z)
    assert check_basis(d, e, Z, g, o) == []
