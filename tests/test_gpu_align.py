"""Device buffers that are not 16-byte aligned. The kernels read and write
whole rows in 16-byte pieces only where the pointer and the row length
allow it and fall back to element accesses elsewhere; both paths must give
the same results bit for bit. Every buffer here is a view one element into
a larger allocation (4-byte or 8-byte aligned only), compared with the same
call on fresh, aligned buffers. Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


def _bits(t):
    import torch
    return t.view(torch.int32 if t.element_size() == 4 else torch.int64)


def _offset(shape, dtype, dev):
    """A contiguous tensor of `shape` starting one element into its storage."""
    import torch
    n = int(np.prod(shape))
    return torch.empty(n + 1, dtype=dtype, device=dev)[1:].view(shape)


# dtype, n, jobz, back-transformation: the register-band, LDS-band and
# producer-consumer kernels, orders with rows of a multiple of four values
# (the 16-byte paths) and one without
CASES = [(np.float32, 16, True, False), (np.float32, 16, True, True), (np.float32, 32, True, False),
         (np.float64, 16, True, False), (np.float64, 32, True, True), (np.float32, 16, False, False),
         (np.float64, 64, True, False), (np.float32, 64, True, True), (np.float32, 128, True, False),
         (np.float64, 128, True, False), (np.float32, 256, True, False), (np.float32, 20, True, False)]


@pytest.mark.parametrize("dt,n,jobz,bt", CASES)
def test_steqr_offset_buffers(dt, n, jobz, bt):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    nb = 300 if n <= 64 else 40
    print("alignment case", dt.__name__, n, jobz, bt, flush=True)
    d, e = W.random_batch(n, nb, dt, salt=3)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dt == np.float32 else torch.float64
    Z = W.random_basis(n, nb, dt, salt=5) if bt else None
    prm = st.make_params(back_transform=bt)
    jz = st.STEQR_V if jobz else st.STEQR_N

    def run(alloc):
        td = alloc((nb, n), tdt, dev)
        te = alloc((nb, n - 1), tdt, dev)
        td.copy_(torch.from_numpy(d))
        te.copy_(torch.from_numpy(e))
        lam = alloc((nb, n), tdt, dev)
        Q = alloc((nb, n, n), tdt, dev) if jobz else None
        if bt:
            Q.copy_(torch.from_numpy(Z))
        info = alloc((nb,), torch.int32, dev)
        rc = st.steqr_batched_ex(td, te, lam, Q, n, nb, jz, st.dtype_code(tdt), info=info,
                                 params=prm)
        assert rc == 0
        torch.cuda.synchronize()
        return lam, Q, info

    lam0, Q0, info0 = run(lambda shape, dtype, dev: torch.empty(shape, dtype=dtype, device=dev))
    lam1, Q1, info1 = run(_offset)
    assert lam1.data_ptr() % 16 != 0
    assert torch.equal(_bits(lam0), _bits(lam1))
    assert torch.equal(info0, info1)
    assert not info0.any()
    if jobz:
        assert torch.equal(_bits(Q0), _bits(Q1))


@pytest.mark.parametrize("name", ["s_f32_n16", "s_f32_n32", "s_f64_n16"])
def test_syev_offset_buffers(name):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    dt, n, _ = W.DENSE_WORKLOADS[name]
    nb = 300
    print("alignment case", name, flush=True)
    A = W.make_dense(name, nb)
    dev = torch.device("cuda:0")
    tdt = torch.float32 if dt == "f32" else torch.float64

    def run(alloc):
        tA = alloc((nb, n, n), tdt, dev)
        tA.copy_(torch.from_numpy(A))
        lam = alloc((nb, n), tdt, dev)
        Q = alloc((nb, n, n), tdt, dev)
        info = alloc((nb,), torch.int32, dev)
        assert st.syev_batched_ex(tA, lam, Q, n, nb, 1, st.dtype_code(tdt), info=info) == 0
        torch.cuda.synchronize()
        return lam, Q, info

    lam0, Q0, info0 = run(lambda shape, dtype, dev: torch.empty(shape, dtype=dtype, device=dev))
    lam1, Q1, info1 = run(_offset)
    assert Q1.data_ptr() % 16 != 0
    assert torch.equal(_bits(lam0), _bits(lam1))
    assert torch.equal(_bits(Q0), _bits(Q1))
    assert torch.equal(info0, info1)
