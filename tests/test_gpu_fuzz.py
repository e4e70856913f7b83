"""Seeded random points of the whole option space against the oracle: order
(1..512, most of them at most 32), precision, jobz, update scheme, shift,
back-transformation, sorting, lanes per problem and band storage (any
combination the library accepts for that order), batch size, and a mix of
ordinary and edge items (splits, graded, zero, scaled, NaN) in one batch;
likewise the values-only bisection and the fused dense solver. Each case is
checked item by item as the other parity tests are. Needs an MI355X; run
with -m gpu."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, check_basis, run_gpu

pytestmark = pytest.mark.gpu

SEEDS = range(192)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import symmetric_tridiagonal_eigensolver_amd  # noqa: F401  (fails loudly if not built)


def _case(seed):
    """(dtype, n, jobz, scheme, shift, bt, sort, batch, lanes, band, d, e, Z)."""
    import symmetric_tridiagonal_eigensolver_amd as st
    g = np.random.default_rng(0xF0CC + seed)
    dt = np.float32 if g.random() < 0.5 else np.float64
    u = g.random()
    if u < 0.65:
        n = int(g.integers(1, 33))
    elif u < 0.9:
        n = int(g.integers(33, 129))
    else:
        n = int(g.integers(129, 513))
    jobz = bool(g.random() < 0.7)
    scheme = int(g.random() < 0.3)
    shift = int(g.random() < 0.3)
    bt = bool(jobz and g.random() < 0.2)
    sort = bool(g.random() < 0.8)
    if n <= 32:
        nb = int(g.integers(1, 258))
    elif n <= 128:
        nb = int(g.integers(1, 34))
    else:
        nb = int(g.integers(1, 3 if jobz else 5))
    # lanes and band storage: the default or a random accepted combination
    code = 0 if dt == np.float32 else 1
    options = [(0, 0)]
    for lanes in (1, 2, 4, 8, 16, 32, 64):
        for band in (0, 1, 2, 3):
            prm = st.make_params(lanes_per_problem=lanes, band_storage=band,
                                 update_scheme=scheme, shift=shift, back_transform=bt)
            try:
                st.steqr_query(n, nb, int(jobz), code, prm)
            except st.SteqrError:
                continue
            options.append((lanes, band))
    lanes, band = options[int(g.integers(0, len(options)))]
    # items: ordinary N(0,1) bands, about one in five an edge item of a
    # random kind
    d, e = W.random_batch(n, nb, dt, salt=seed, cfg=7)
    for b in range(nb):
        if g.random() < 0.2:
            kind = int(g.integers(0, 5))
            de, ee = W.edge_batch(kind, n, 1, dt, salt=1000 * seed + b)
            d[b], e[b] = de[0], ee[0]
    Z = W.random_basis(n, nb, dt, salt=seed) if bt else None
    return dt, n, jobz, scheme, shift, bt, sort, nb, lanes, band, d, e, Z


def _sorted(lam, Q, info):
    """Converged items in ascending order (NaN last, ties by index), Q's
    columns permuted alike; failed items as they are (never sorted)."""
    lam = lam.copy()
    Q = None if Q is None else Q.copy()
    for b in np.nonzero(info == 0)[0]:
        k = np.argsort(lam[b], kind="stable")
        lam[b] = lam[b][k]
        if Q is not None:
            Q[b] = Q[b][:, k]
    return lam, Q, info


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    dt, n, jobz, scheme, shift, bt, sort, nb, lanes, band, d, e, Z = _case(seed)
    print("fuzz case seed=%d %s n=%d jobz=%s scheme=%d shift=%d bt=%s sort=%s batch=%d "
          "lanes=%d band=%d" % (seed, dt.__name__, n, jobz, scheme, shift, bt, sort, nb, lanes,
                                band), flush=True)
    g = run_gpu(d, e, jobz, sort=sort, lanes=lanes, band=band, scheme=scheme, shift=shift, Z=Z)
    if not sort:
        g = _sorted(*g)
    o = oracle.steqr(d, e, jobz, threads=8, scheme=scheme, shift=shift, Z=Z)
    if bt:
        assert check_basis(d, e, Z, g, o) == []
    else:
        assert check(d, e, g, o, jobz) == []


def _mixed_items(g, n, nb, dt, seed):
    d, e = W.random_batch(n, nb, dt, salt=seed, cfg=9)
    for b in range(nb):
        if g.random() < 0.2:
            kind = int(g.integers(0, 5))
            de, ee = W.edge_batch(kind, n, 1, dt, salt=2000 * seed + b)
            d[b], e[b] = de[0], ee[0]
    return d, e


@pytest.mark.parametrize("seed", range(64))
def test_random_bisection(seed):
    """Values-only bisection at random orders 1..512 and batches with mixed
    edge items, against the oracle's bisection."""
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    g = np.random.default_rng(0xB15E + seed)
    dt = np.float32 if g.random() < 0.5 else np.float64
    u = g.random()
    n = int(g.integers(1, 65)) if u < 0.7 else int(g.integers(65, 513))
    nb = int(g.integers(1, 258)) if n <= 64 else int(g.integers(1, 17))
    print("fuzz bisection seed=%d %s n=%d batch=%d" % (seed, dt.__name__, n, nb), flush=True)
    d, e = _mixed_items(g, n, nb, dt, seed)
    dev = torch.device("cuda:0")
    lam, _, info = st.solve(torch.from_numpy(d).to(dev), torch.from_numpy(e).to(dev), False,
                            info=True, method=1)
    torch.cuda.synchronize()
    gpu = (lam.cpu().numpy(), None, info.cpu().numpy())
    lo, io = oracle.stebz(d, e, threads=8)
    assert check(d, e, gpu, (lo, None, io), False) == []


@pytest.mark.parametrize("seed", range(64))
def test_random_syev(seed):
    """The fused dense solver at random orders 1..32, batches, shifts,
    sorting and lanes, with zero, diagonal, tridiagonal and scaled items
    among random symmetric ones, against the oracle's syev."""
    import symmetric_tridiagonal_eigensolver_amd as st
    from parity import check_dense, run_gpu_syev
    g = np.random.default_rng(0x5E7 + seed)
    dt = np.float32 if g.random() < 0.5 else np.float64
    n = int(g.integers(1, 33))
    jobz = bool(g.random() < 0.7) and (dt == np.float32 or n <= st.SYEV_MAX_N_F64_V)
    shift = int(g.random() < 0.3)
    sort = bool(g.random() < 0.8)
    nb = int(g.integers(1, 301))
    code = 0 if dt == np.float32 else 1
    options = [0]
    for lanes in (1, 2, 4, 8, 16, 32, 64):
        try:
            st.syev_query(n, nb, int(jobz), code, st.make_params(lanes_per_problem=lanes,
                                                                shift=shift))
        except st.SteqrError:
            continue
        options.append(lanes)
    lanes = options[int(g.integers(0, len(options)))]
    print("fuzz syev seed=%d %s n=%d jobz=%s shift=%d sort=%s batch=%d lanes=%d"
          % (seed, dt.__name__, n, jobz, shift, sort, nb, lanes), flush=True)
    A = W.random_symmetric(n, nb, np.float64, salt=seed, cfg=10)
    for b in range(nb):
        r = g.random()
        if r < 0.04:
            A[b] = 0.0
        elif r < 0.08:
            A[b] = np.diag(np.diag(A[b]))
        elif r < 0.12:
            A[b] = np.triu(np.tril(A[b], 1), -1)
        elif r < 0.16:
            A[b] *= 10.0 ** (int(g.integers(-12, 13)))
    A = np.ascontiguousarray(A.astype(dt))
    gpu = run_gpu_syev(A, jobz, sort=sort, lanes=lanes, shift=shift)
    o = oracle.syev(A, jobz, threads=8, shift=shift, sort=sort)
    assert check_dense(A, gpu, o, jobz, sort=sort) == []
