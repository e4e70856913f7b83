"""Batches whose arrays have more than 2^31 elements: every offset into d,
e, lambda, Q and info is computed in 64 bits. The inputs are drawn on the
device by torch's seeded generator (N(0,1) bands); the last items and a
spread sample are copied back and checked against the oracle, and the
status of every item is checked on the device. Needs an MI355X with about
20 GB free; run with -m gpu."""
import numpy as np
import pytest

import oracle
from parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


# (order, jobz, batch): values only at order 16 puts d past 2^31 elements,
# order 4 with eigenvectors puts Q past it
CASES = [(16, False, (1 << 27) + 3), (4, True, (1 << 27) + 5)]


@pytest.mark.parametrize("n,jobz,nb", CASES)
def test_batch_beyond_int32_offsets(n, jobz, nb):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    print("huge batch case n=%d jobz=%s batch=%d" % (n, jobz, nb), flush=True)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202 + n)
    td = torch.randn((nb, n), generator=gen, device=dev, dtype=torch.float32)
    te = torch.randn((nb, n - 1), generator=gen, device=dev, dtype=torch.float32)
    lam, Q, info = st.solve(td, te, jobz, info=True)
    torch.cuda.synchronize()
    assert (td.numel() if not jobz else Q.numel()) > (1 << 31)
    assert int(info.abs().max().item()) == 0
    items = np.unique(np.concatenate([np.linspace(0, nb - 1, 256).astype(np.int64),
                                      np.arange(nb - 64, nb)]))
    idx = torch.from_numpy(items).to(dev)
    d = td.index_select(0, idx).cpu().numpy()
    e = te.index_select(0, idx).cpu().numpy()
    g = (lam.index_select(0, idx).cpu().numpy(),
         Q.index_select(0, idx).cpu().numpy() if jobz else None,
         info.index_select(0, idx).cpu().numpy())
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []
