"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs. Needs an MI355X; run with -m gpu."""
import numpy as np
import pytest

import oracle
import validate as V
import workloads as W
from parity import check, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


def _case(w, jobz, batch):
    print("case %s jobz=%s batch=%d" % (w.name, jobz, batch), flush=True)


SMALL = 1000 + 13  # several workgroups and a ragged tail for every P


@pytest.mark.parametrize("wname", W.SMALL_BATCH_WORKLOADS)
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_workload_small_batch(wname, jobz):
    w = W.WORKLOADS[wname]
    _case(w, jobz, SMALL)
    d, e = W.make_batch(w, SMALL)
    g = run_gpu(d, e, jobz)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("wname", list(W.WORKLOADS))
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_workload_full_size(wname, jobz):
    """Full batch in the default launch configuration (the one the
    benchmark times); the oracle checks a spread sample plus the tail, and
    properties that hold at any size are checked on every item."""
    w = W.WORKLOADS[wname]
    _case(w, jobz, w.batch)
    d, e = W.make_batch(w)
    g = run_gpu(d, e, jobz)
    nb = w.batch
    # at order 512 (about a second of oracle time per matrix with
    # eigenvectors) 24 spread items and the last 8
    ns, nt = (384, 40) if w.n <= 256 else (24, 8)
    items = np.unique(np.concatenate([np.linspace(0, nb - 1, ns).astype(int),
                                      np.arange(nb - nt, nb)]))
    o = oracle.steqr(d[items], e[items], jobz, threads=8)
    assert check(d, e, g, o, jobz, items=items) == []
    lam, Q, info = g
    finite = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    assert not info[finite].any()
    assert np.all(info[~finite] > 0)
    ok = info == 0
    tol = V.tol_of(d.dtype, w.n)
    assert np.all(np.diff(lam[ok], axis=1) >= 0)
    tn = V.tnorm1(d[ok], e[ok])
    assert np.all(np.abs(lam[ok].astype(np.float64).sum(1)
                         - d[ok].astype(np.float64).sum(1)) <= w.n * tol * tn)
    if jobz:
        assert V.band_residual(d[ok], e[ok], lam[ok], Q[ok]).max() <= tol
        assert V.orthogonality(Q[ok]).max() <= tol


@pytest.mark.parametrize("wname,batch,P", [("c2_f32_n16", 65536, 1), ("c4_f32_n32", 65536, 2),
                                           ("c4_f32_n32", 131072, 1), ("w_f32_n128", 16384, 8)])
def test_values_only_large_batch_default(wname, batch, P):
    """Values only at two and four times the configuration's batch, where
    the default launch takes fewer lanes per problem: a spread sample and
    the tail against the oracle, properties on every item."""
    import symmetric_tridiagonal_eigensolver_amd as st
    w = W.WORKLOADS[wname]
    _case(w, False, batch)
    assert st.steqr_query(w.n, batch, 0, 0)["lanes_per_problem"] == P
    d, e = W.make_batch(w, batch)
    g = run_gpu(d, e, False)
    items = np.unique(np.concatenate([np.linspace(0, batch - 1, 512).astype(int),
                                      np.arange(batch - 64, batch)]))
    o = oracle.steqr(d[items], e[items], False, threads=8)
    assert check(d, e, g, o, False, items=items) == []
    lam, _, info = g
    finite = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    assert not info[finite].any()
    assert np.all(info[~finite] > 0)
    ok = info == 0
    tol = V.tol_of(d.dtype, w.n)
    assert np.all(np.diff(lam[ok], axis=1) >= 0)
    tn = V.tnorm1(d[ok], e[ok])
    assert np.all(np.abs(lam[ok].astype(np.float64).sum(1)
                         - d[ok].astype(np.float64).sum(1)) <= w.n * tol * tn)


LANE_CASES = [
    # dtype, n, jobz, lanes
    (np.float32, 4, True, 4), (np.float32, 4, True, 2), (np.float32, 4, True, 1),
    (np.float32, 8, True, 8), (np.float32, 8, True, 4), (np.float32, 8, True, 2),
    (np.float32, 16, True, 16), (np.float32, 16, True, 8), (np.float32, 16, True, 4),
    (np.float32, 32, True, 32), (np.float32, 32, True, 16),
    (np.float32, 4, False, 1), (np.float32, 8, False, 1), (np.float32, 16, False, 4),
    (np.float32, 16, False, 1), (np.float32, 32, False, 4), (np.float32, 32, False, 1),
    (np.float64, 4, True, 2), (np.float64, 8, True, 4), (np.float64, 16, True, 8),
    (np.float64, 4, False, 1), (np.float64, 8, False, 1),
    (np.float64, 16, False, 1), (np.float64, 32, False, 1),
    (np.float32, 16, True, 2), (np.float32, 8, True, 1), (np.float32, 8, False, 2),
    (np.float32, 16, False, 2), (np.float32, 32, False, 2),
    (np.float64, 8, True, 2), (np.float64, 4, True, 4), (np.float64, 8, False, 2),
    (np.float32, 64, True, 64), (np.float32, 64, False, 64), (np.float64, 64, False, 64),
    (np.float32, 33, True, 64),
    (np.float64, 16, False, 2), (np.float64, 32, False, 2),
]


LANE_CASES = [c + (1,) for c in LANE_CASES if c[1] <= 32] + [c + (2,) for c in LANE_CASES
                                                              if c[1] > 32]
# band in LDS (chunked kernel variant)
LANE_CASES += [
    (np.float32, 16, True, 8, 2), (np.float32, 16, True, 4, 2), (np.float32, 16, True, 2, 2),
    (np.float32, 32, True, 16, 2), (np.float32, 32, True, 8, 2),
    (np.float64, 16, True, 8, 2), (np.float64, 16, True, 4, 2), (np.float64, 32, True, 16, 2),
    (np.float32, 12, True, 4, 2), (np.float64, 27, True, 16, 2),
    # compiled order 12 (double with eigenvectors, orders 9..12)
    (np.float64, 12, True, 4, 2), (np.float64, 9, True, 4, 2), (np.float64, 12, True, 4, 1),
    (np.float64, 10, True, 4, 1),
]
# the producer's algorithm alone, several problems per wavefront (orders
# 33..64 without eigenvectors)
LANE_CASES += [
    (np.float32, 64, False, 4, 2), (np.float32, 64, False, 8, 2), (np.float32, 64, False, 16, 2),
    (np.float64, 64, False, 4, 2), (np.float64, 64, False, 8, 2), (np.float64, 64, False, 16, 2),
    (np.float32, 41, False, 8, 2), (np.float64, 59, False, 8, 2),
]
# producer and consumer wavefronts (orders 33..64 with eigenvectors)
LANE_CASES += [
    (np.float32, 64, True, 16, 3), (np.float32, 64, True, 8, 3), (np.float64, 64, True, 4, 3),
    (np.float64, 33, True, 16, 3), (np.float32, 48, True, 16, 3), (np.float64, 57, True, 4, 3),
]


# Variants that need more than 256 registers per lane are not built (the
# build rejects them): the LDS-band kernel in double at order 32 with 8 lanes
# per problem returned wrong eigenvectors on the GPU in one build, with
# correct eigenvalues, and its cause was not found; the register-band
# kernels at these lanes and the one-problem-per-wavefront kernel in double
# with eigenvectors share the register budget. Kept as skipped cases.
OVER_BUDGET = [
    (np.float64, 32, True, 8, 2), (np.float32, 32, True, 4, 2),
    (np.float32, 32, True, 8, 1), (np.float64, 16, True, 4, 1), (np.float64, 32, True, 16, 1),
    (np.float64, 32, True, 32, 1), (np.float64, 64, True, 64, 2), (np.float64, 48, True, 64, 2),
]
LANE_CASES += [pytest.param(*c, marks=pytest.mark.skip(
    reason="needs more than 256 registers per lane: not built (wrong eigenvectors in one "
           "build of double order 32 at 8 lanes, cause not found)")) for c in OVER_BUDGET]


@pytest.mark.parametrize("dt,n,jobz,lanes,band", LANE_CASES,
                         ids=lambda v: v.__name__ if isinstance(v, type) else str(v))
def test_lanes_per_problem_variants(dt, n, jobz, lanes, band):
    d, e = W.random_batch(n, 777, dt, salt=21)
    print("lanes case", dt.__name__, n, jobz, lanes, band, flush=True)
    g = run_gpu(d, e, jobz, lanes=lanes, band=band)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, g, o, jobz) == []


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("band", [1, 2], ids=["regs", "lds"])
def test_band_storage_variants_on_edge_items(dt, band):
    # double with eigenvectors keeps the band in registers up to order 16
    orders = (9, 16) if (dt == np.float64 and band == 1) else (9, 16, 32)
    for kind in range(5):
        for n in orders:
            d, e = W.edge_batch(kind, n, 70, dt, salt=3)
            g = run_gpu(d, e, True, band=band)
            o = oracle.steqr(d, e, True)
            assert check(d, e, g, o, True) == [], (W.EDGE_NAMES[kind], n)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_every_order_up_to_64(dt, jobz):
    for n in range(1, 65):
        d, e = W.random_batch(n, 67, dt, salt=n)
        print("order", n, flush=True)
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz)
        assert check(d, e, g, o, jobz) == [], "n=%d" % n


@pytest.mark.parametrize("kind", range(5), ids=W.EDGE_NAMES)
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [3, 4, 16, 32, 40, 64])
def test_edge_items(kind, dt, n):
    d, e = W.edge_batch(kind, n, 130, dt)
    print("edge", W.EDGE_NAMES[kind], dt.__name__, n, flush=True)
    for jobz in (True, False):
        g = run_gpu(d, e, jobz)
        o = oracle.steqr(d, e, jobz)
        assert check(d, e, g, o, jobz) == [], (W.EDGE_NAMES[kind], jobz)
    if kind == W.EDGE_ZERO:
        assert np.all(g[0] == 0)
    if kind == W.EDGE_NAN:
        assert np.all(g[2] > 0)


def test_scaled_items_match_unscaled_twins():
    n = 32
    d, e = W.edge_batch(W.EDGE_SCALED, n, 64, np.float64)
    f = np.where(np.arange(64) % 2 == 0, 1e18, 1e-18)
    for dt in (np.float32, np.float64):
        lam, _, info = run_gpu(d.astype(dt), e.astype(dt), False)
        base, _, binfo = run_gpu((d / f[:, None]).astype(dt), (e / f[:, None]).astype(dt), False)
        assert not info.any() and not binfo.any()
        err = V.sorted_err(lam.astype(np.float64) / f[:, None], base, d / f[:, None],
                           e / f[:, None])
        assert err.max() <= V.tol_of(dt, n)


def test_nan_confined_to_block():
    n = 12
    d, e = W.random_batch(n, 8, np.float64, salt=3)
    e[:, 5] = 0.0
    d[:, 8] = np.nan
    g = run_gpu(d, e, True)
    o = oracle.steqr(d, e, True)
    assert check(d, e, g, o, True) == []
    assert np.all(g[2] == 5)
    assert np.all(np.isfinite(g[0][:, :6])) and np.all(np.isnan(g[0][:, 6:]))


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_budget_exhaustion(dt):
    d, e = W.random_batch(16, 100, dt, salt=8)
    lam, _, info = run_gpu(d, e, False, max_sweeps_per_n=-1)
    ol, _, oinfo, _ = oracle.steqr(d, e, False, max_sweeps_per_n=0)
    assert np.array_equal(info, oinfo) and np.all(info > 0)
    assert np.array_equal(lam, d)
    lam1, _, info1 = run_gpu(d, e, True, max_sweeps_per_n=1)
    o1 = oracle.steqr(d, e, True, max_sweeps_per_n=1)
    assert np.array_equal(info1 > 0, o1[2] > 0)


def test_unsorted_output():
    d, e = W.random_batch(13, 300, np.float32, salt=4)
    lam, Q, info = run_gpu(d, e, True, sort=False)
    slam, _, _ = run_gpu(d, e, True)
    assert not info.any()
    assert np.array_equal(np.sort(lam, axis=1), slam)
    assert V.band_residual(d, e, lam, Q).max() <= V.tol_of(np.float32, 13)


def test_deterministic_and_launch_shape_independent():
    d, e = W.make_batch(W.WORKLOADS["c2_f32_n16"], 4096)
    a = run_gpu(d, e, True)
    b = run_gpu(d, e, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for waves in (1, 2, 4):
        c = run_gpu(d, e, True, waves=waves)
        for x, y in zip(a, c):
            assert np.array_equal(x, y)


def test_checker_is_not_vacuous():
    d, e = W.random_batch(16, 200, np.float32, salt=6)
    g = run_gpu(d, e, True)
    o = oracle.steqr(d, e, True)
    assert check(d, e, g, o, True) == []
    lam, Q, info = g
    bad = lam.copy()
    bad[7, 3] += 1e-3 * V.tnorm1(d, e)[7]
    assert check(d, e, (bad, Q, info), o, True)
    badq = Q.copy()
    badq[9, :, [2, 3]] = badq[9, :, [3, 2]]
    assert check(d, e, (lam, badq, info), o, True)
    badi = info.copy()
    badi[0] = 1
    assert check(d, e, (lam, Q, badi), o, True)


def test_non_default_stream():
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    d, e = W.random_batch(16, 500, np.float32, salt=1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        td = torch.from_numpy(d).cuda()
        te = torch.from_numpy(e).cuda()
        lam, Q = st.solve(td, te, True)
    s.synchronize()
    o = oracle.steqr(d, e, True)
    g = (lam.cpu().numpy(), Q.cpu().numpy(), np.zeros(500, np.int32))
    assert check(d, e, g, o, True) == []


def test_accuracy_margins_report():
    """Report (and bound) error / tolerance on every configuration: the
    largest eigenvalue, residual and orthogonality error as a fraction of
    the 16 n eps acceptance bound."""
    for wname in W.SMALL_BATCH_WORKLOADS:
        w = W.WORKLOADS[wname]
        d, e = W.make_batch(w, 2048)
        g = run_gpu(d, e, True)
        o = oracle.steqr(d, e, True, threads=8)
        ok = (g[2] == 0) & (o[2] == 0)
        tol = V.tol_of(d.dtype, w.n)
        ev = V.sorted_err(g[0][ok], o[0][ok], d[ok], e[ok]).max() / tol
        rs = V.band_residual(d[ok], e[ok], g[0][ok], g[1][ok]).max() / tol
        og = V.orthogonality(g[1][ok]).max() / tol
        print("margin %-12s eig %.3f  residual %.3f  orth %.3f" % (wname, ev, rs, og), flush=True)
        assert max(ev, rs, og) <= 1.0


@pytest.mark.parametrize("wname,jobz", [("c2_f32_n16", True), ("c4_f64_n32", False),
                                        ("c3_f64_n12", True)])
def test_plain_entry_point(wname, jobz):
    """The 9-argument steqr_batched (no status, no params) on a full
    workload batch: the same launch as steqr_batched_ex with defaults, so
    its outputs are bit-identical to that call's; a sample checked against
    the oracle."""
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    w = W.WORKLOADS[wname]
    _case(w, jobz, w.batch)
    d, e = W.make_batch(w)
    dev = torch.device("cuda:0")
    td, te = torch.from_numpy(d).to(dev), torch.from_numpy(e).to(dev)
    lam = torch.empty_like(td)
    Q = torch.empty((w.batch, w.n, w.n), dtype=td.dtype, device=dev) if jobz else None
    rc = st.steqr_batched(td, te, lam, Q, w.n, w.batch, st.STEQR_V if jobz else st.STEQR_N,
                          st.dtype_code(td.dtype))
    assert rc == 0
    torch.cuda.synchronize()
    g = (lam.cpu().numpy(), None if Q is None else Q.cpu().numpy())
    ref = run_gpu(d, e, jobz)
    assert np.array_equal(g[0], ref[0], equal_nan=True)
    if jobz:
        assert np.array_equal(g[1], ref[1], equal_nan=True)
    items = np.unique(np.concatenate([np.linspace(0, w.batch - 1, 256).astype(int),
                                      np.arange(w.batch - 16, w.batch)]))
    o = oracle.steqr(d[items], e[items], jobz, threads=8)
    assert check(d, e, (g[0], g[1], ref[2]), o, jobz, items=items) == []


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [16, 32])
@pytest.mark.parametrize("top", [False, True], ids=["small_end_bottom", "small_end_top"])
def test_graded_keeps_relative_accuracy(dt, n, top):
    """Graded items converge their small end first ("STEQR: the CTA
    tridiagonal solver", QL versus QR), which keeps the small eigenvalues
    accurate relative to their size in both orientations: within 2^-6
    (float) or 2^-30 (double) of long-double Sturm values, where the
    opposite rule loses all digits in float at these orders (1.4 at order
    16) and 2.8e-9 or more in double (oracle measurements). Float keeps no
    fixed number of digits on graded input (the pages call the method
    normwise accurate), hence the loose float bound; the usual parity with
    the oracle is checked too."""
    d, e = W.edge_batch(W.EDGE_NAMES.index("graded"), n, 333, np.float64)
    if top:
        d, e = d[:, ::-1].copy(), e[:, ::-1].copy()
    d, e = d.astype(dt), e.astype(dt)
    g = run_gpu(d, e, True)
    o = oracle.steqr(d, e, True, threads=8)
    assert check(d, e, g, o, True) == []
    ref = np.sort(V.sturm_eigvals(d[:64], e[:64]).astype(np.float64), axis=1)
    rel = np.abs(np.sort(g[0][:64].astype(np.float64), axis=1) - ref) / np.abs(ref)
    assert rel.max() <= (2.0 ** -6 if dt == np.float32 else 2.0 ** -30)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [2, 4, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("jobz", [True, False], ids=["V", "N"])
def test_infinite_entries(n, dt, jobz):
    """Items with +-inf in d or e among ordinary ones: the same status,
    NaN positions and values as the oracle (the block scaling turns an
    infinite norm into NaN entries, as on the CPU)."""
    print("infinite entries", n, dt.__name__, jobz, flush=True)
    nb = 40 if n <= 64 else 12
    d, e = W.random_batch(n, nb, dt, salt=51)
    g = np.random.default_rng(n)
    for b in range(0, nb, 3):
        if n > 1 and g.random() < 0.5:
            e[b, int(g.integers(0, n - 1))] = np.inf if g.random() < 0.5 else -np.inf
        else:
            d[b, int(g.integers(0, n))] = np.inf if g.random() < 0.5 else -np.inf
    gpu = run_gpu(d, e, jobz)
    o = oracle.steqr(d, e, jobz, threads=8)
    assert check(d, e, gpu, o, jobz) == []
