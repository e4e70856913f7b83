"""The C entry point under HIP graph capture and from concurrent host
threads. The library only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronisation, no state), so a call can be
captured once and replayed, every replay reproducing the eager result bit
for bit with unrelated eager work and host synchronisations between the
replays, and calls from two threads on two streams give the results of the
same calls made in sequence. Needs an MI355X; run with -m gpu."""
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


def test_concurrent_streams_and_threads_match_sequential():
    """The library keeps no state: calls from two host threads, each on its
    own stream, give the same results as the same calls made one after the
    other on one stream."""
    import threading

    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    dev = torch.device("cuda:0")
    cases = []
    for wname, jobz, nb in (("c2_f32_n16", True, 4096), ("c4_f64_n32", True, 2048),
                            ("c2_f32_n8", False, 8192), ("w_f32_n128", True, 256)):
        w = W.WORKLOADS[wname]
        d, e = W.make_batch(w, nb)
        cases.append((w.n, jobz, torch.from_numpy(d).to(dev), torch.from_numpy(e).to(dev)))

    def run(case, stream):
        n, jobz, td, te = case
        nb = td.shape[0]
        lam = torch.empty_like(td)
        Q = torch.empty((nb, n, n), dtype=td.dtype, device=dev) if jobz else None
        info = torch.empty(nb, dtype=torch.int32, device=dev)
        rc = st.steqr_batched_ex(td, te, lam, Q, n, nb, st.STEQR_V if jobz else st.STEQR_N,
                                 st.dtype_code(td.dtype), stream, info=info)
        assert rc == 0
        return lam, Q, info

    ref = [run(c, torch.cuda.current_stream()) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = [None] * len(cases)

    def worker(k):
        s = streams[k % 2]
        with torch.cuda.stream(s):
            for i in range(k % 2, len(cases), 2):
                out[i] = run(cases[i], s)
        s.synchronize()

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for (l0, q0, i0), (l1, q1, i1) in zip(ref, out):
        assert torch.equal(_bits(l0), _bits(l1)) and torch.equal(i0, i1)
        if q0 is not None:
            assert torch.equal(_bits(q0), _bits(q1))
