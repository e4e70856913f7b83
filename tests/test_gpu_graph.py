"""HIP graph capture of the C entry point. The library only enqueues kernels
on the caller's stream (no allocation, no memset, no host synchronisation),
so a call can be captured once and replayed: every replay must reproduce
the eager result bit for bit, with unrelated eager work (refilling the
outputs) and host synchronisations between the replays. Needs an MI355X;
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


def _bits(t):
    import torch
    return t.view(torch.int32 if t.element_size() == 4 else torch.int64)


@pytest.mark.parametrize("wname,jobz", [("c2_f32_n16", True), ("c4_f64_n32", False),
                                        ("c5_f64_n64", True), ("w_f32_n256", True)])
def test_graph_replays_match_eager(wname, jobz):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    w = W.WORKLOADS[wname]
    nb = min(w.batch, 2048)
    print("graph case", wname, jobz, nb, flush=True)
    d, e = W.make_batch(w, nb)
    dev = torch.device("cuda:0")
    td, te = torch.from_numpy(d).to(dev), torch.from_numpy(e).to(dev)
    n = w.n
    dcode = st.dtype_code(td.dtype)
    jz = st.STEQR_V if jobz else st.STEQR_N

    def outputs():
        lam = torch.empty_like(td)
        Q = torch.empty((nb, n, n), dtype=td.dtype, device=dev) if jobz else None
        info = torch.empty(nb, dtype=torch.int32, device=dev)
        return lam, Q, info

    lam0, Q0, info0 = outputs()
    assert st.steqr_batched_ex(td, te, lam0, Q0, n, nb, jz, dcode, info=info0) == 0
    torch.cuda.synchronize()

    lam, Q, info = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch outside the capture
        assert st.steqr_batched_ex(td, te, lam, Q, n, nb, jz, dcode, info=info) == 0
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rc = st.steqr_batched_ex(td, te, lam, Q, n, nb, jz, dcode, info=info)
    assert rc == 0
    for k in range(3):
        lam.fill_(float("nan"))
        info.fill_(-7)
        if Q is not None:
            Q.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(lam), _bits(lam0)), k
        assert torch.equal(info, info0), k
        if jobz:
            assert torch.equal(_bits(Q), _bits(Q0)), k
    assert np.all(info0.cpu().numpy()[np.isfinite(d).all(1) & np.isfinite(e).all(1)] == 0)
