"""Every launch shape computes the same bits. The kernel families (band in
registers or LDS, producer and consumer wavefronts, one problem per
wavefront) and their lanes per problem differ only in which lanes do
which part of the work: the arithmetic of each problem, its order and its
rounding are the same, so the eigenvalues, Q and the status are bit-for-bit
equal across every (lanes per problem, band storage) the library accepts
for an order. This is what lets the default lanes depend on the batch.
(The fused dense solver is not covered: its Householder reduction sums
each dot product over the lane's own rows and then across the chunk's
lanes, so its last bits depend on the lanes per problem.) Needs an MI355X;
run with -m gpu."""
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


def _shapes(n, nb, jobz, code, scheme):
    import symmetric_tridiagonal_eigensolver_amd as st
    out = []
    for lanes in (1, 2, 4, 8, 16, 32, 64):
        for band in (1, 2, 3):
            try:
                q = st.steqr_query(n, nb, int(jobz), code,
                                   st.make_params(lanes_per_problem=lanes, band_storage=band,
                                                  update_scheme=scheme))
            except st.SteqrError:
                continue
            key = (q["lanes_per_problem"], q["band_storage"])
            if key not in out:
                out.append(key)
    return out


@pytest.mark.parametrize("scheme", [0, 1], ids=["EXP", "PG"])
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [4, 8, 12, 16, 27, 32, 48, 64, 100, 128, 200, 256])
def test_launch_shapes_bit_identical(n, dt, jobz, scheme):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    nb = 300 if n <= 64 else (24 if n <= 128 else 8)
    code = 0 if dt == np.float32 else 1
    shapes = _shapes(n, nb, jobz, code, scheme)
    print("launch shapes n=%d %s jobz=%s scheme=%d: %s" % (n, dt.__name__, jobz, scheme, shapes),
          flush=True)
    if len(shapes) < 2:
        pytest.skip("one launch shape at this order")
    # ordinary items and every edge kind
    d, e = W.random_batch(n, nb, dt, salt=21)
    for b in range(9, nb, 10):
        de, ee = W.edge_batch((b // 10) % 5, n, 1, dt, salt=b)
        d[b], e[b] = de[0], ee[0]
    dev = torch.device("cuda:0")
    td, te = torch.from_numpy(d).to(dev), torch.from_numpy(e).to(dev)
    iv = torch.int32 if dt == np.float32 else torch.int64
    ref = None
    for lanes, band in shapes:
        lam, Q, info = st.solve(td, te, jobz, info=True, lanes_per_problem=lanes,
                                band_storage=band, update_scheme=scheme)
        torch.cuda.synchronize()
        cur = (lam.view(iv).cpu(), None if Q is None else Q.view(iv).cpu(), info.cpu())
        if ref is None:
            ref = cur
            continue
        assert torch.equal(cur[0], ref[0]), (lanes, band)
        assert torch.equal(cur[2], ref[2]), (lanes, band)
        if jobz:
            assert torch.equal(cur[1], ref[1]), (lanes, band)

