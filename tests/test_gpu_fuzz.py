"""Seeded random points of the whole option space against the oracle: order
(1..512, most of them at most 32), precision, jobz, update scheme, shift,
back-transformation, sorting, lanes per problem and band storage (any
combination the library accepts for that order), batch size, and a mix of
ordinary and edge items (splits, graded, zero, scaled, NaN) in one batch.
Each case is checked item by item as the other parity tests are. Needs an
MI355X; run with -m gpu."""
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
