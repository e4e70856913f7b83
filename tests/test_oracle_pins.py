"""The CPU oracle pinned to what the pages and the mathematics fix.

Nothing here compares the oracle with itself or retypes its formulas:
every check is a closed form, a bisection in higher precision, an
invariant, a library routine on the dense matrix, or a stated special case.
"""
import math
import os

import numpy as np
import pytest

import oracle_pins as P
import validate as V
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


# ---------------------------------------------------------------- constants

def test_constants_exact(oracle_mod):
    c32 = oracle_mod.constants(np.float32)
    assert c32["eps"] == 2.0 ** -24
    assert c32["safmin"] == 2.0 ** -126
    assert c32["ssfmin"] == 2.0 ** -15          # sqrt(2^-126) / 2^-48
    assert c32["ssfmax"] == float(np.float32(2.0 ** 63 / 3))
    assert c32["eps2"] == 2.0 ** -48
    c64 = oracle_mod.constants(np.float64)
    assert c64["eps"] == 2.0 ** -53
    assert c64["safmin"] == 2.0 ** -1022
    assert c64["ssfmin"] == 2.0 ** -405          # sqrt(2^-1022) / 2^-106
    assert c64["ssfmax"] == 2.0 ** 511 / 3
    assert c64["eps2"] == 2.0 ** -106


# ---------------------------------------------------------------- building blocks

@pytest.mark.parametrize("pin", [P.pin_lartg, P.pin_shift, P.pin_sym2x2, P.pin_sweep],
                         ids=lambda p: p.__name__)
def test_building_block_pins(oracle_mod, pin):
    assert pin(oracle_mod) == []


def test_pg_sweep_pins(oracle_mod):
    """The PG form of the sweep against the same explicit shifted QR step."""
    assert P.pin_sweep(oracle_mod, scheme=1) == []


@pytest.mark.parametrize("shift", [0, 1], ids=["lapack_shift", "closed_shift"])
@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
def test_solve_pins_full(oracle_mod, scheme, shift):
    assert P.pin_solve(oracle_mod, quick=False, scheme=scheme, shift=shift) == []


@pytest.mark.parametrize("shift", [0, 1], ids=["lapack_shift", "closed_shift"])
@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
def test_back_transform_pins(oracle_mod, scheme, shift):
    assert P.pin_back_transform(oracle_mod, quick=False, scheme=scheme, shift=shift) == []


@pytest.mark.parametrize("scheme,shift", [(0, 0), (1, 1)])
def test_large_order_pins(oracle_mod, scheme, shift):
    assert P.pin_large_orders(oracle_mod, scheme=scheme, shift=shift) == []


@pytest.mark.parametrize("scheme,shift", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("pin", [P.pin_direction, P.pin_block2], ids=["direction", "block2"])
def test_direction_and_2x2_pins(oracle_mod, pin, scheme, shift):
    assert pin(oracle_mod, quick=False, scheme=scheme, shift=shift) == []


@pytest.mark.parametrize("pin", [P.pin_larfg, P.pin_sytrd, P.pin_syev, P.pin_stebz],
                         ids=lambda p: p.__name__)
def test_dense_front_end_pins(oracle_mod, pin):
    assert pin(oracle_mod) == []


@pytest.mark.parametrize("wname", ["c2_f32_n16", "c4_f64_n32", "c5_f64_n64"])
def test_closed_and_lapack_shift_agree(oracle_mod, wname):
    """The two forms of the shift give the same eigenvalue of the trailing
    2x2 up to rounding, hence the same eigenvalues to the tolerance and
    nearly the same sweep counts."""
    w = W.WORKLOADS[wname]
    d, e = W.make_batch(w, 96)
    ok = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    l0, _, i0, s0 = oracle_mod.steqr(d, e, False)
    l1, Q1, i1, s1 = oracle_mod.steqr(d, e, True, shift=1)
    assert np.array_equal(i0 > 0, i1 > 0)
    tol = V.tol_of(d.dtype, w.n)
    assert V.sorted_err(l1[ok], l0[ok].astype(np.float64), d[ok], e[ok]).max() <= tol
    assert V.band_residual(d[ok], e[ok], l1[ok], Q1[ok]).max() <= tol
    assert V.orthogonality(Q1[ok]).max() <= tol
    assert abs(int(s1[ok, 0].sum()) - int(s0[ok, 0].sum())) <= 0.02 * s0[ok, 0].sum()


@pytest.mark.parametrize("wname", ["c2_f32_n16", "c3_f64_n12", "c4_f64_n32"])
def test_pg_and_exp_agree(oracle_mod, wname):
    """The two update schemes are equivalent forms of one implicit step: on
    the same inputs their eigenvalues agree within the tolerance and their
    sweep counts agree (up to rounding-decided deflations)."""
    w = W.WORKLOADS[wname]
    d, e = W.make_batch(w, 128)
    ok = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    l0, _, i0, s0 = oracle_mod.steqr(d, e, False)
    l1, Q1, i1, s1 = oracle_mod.steqr(d, e, True, scheme=1)
    assert np.array_equal(i0 > 0, i1 > 0)
    tol = V.tol_of(d.dtype, w.n)
    assert V.sorted_err(l1[ok], l0[ok].astype(np.float64), d[ok], e[ok]).max() <= tol
    assert V.band_residual(d[ok], e[ok], l1[ok], Q1[ok]).max() <= tol
    assert V.orthogonality(Q1[ok]).max() <= tol
    assert abs(int(s1[ok, 0].sum()) - int(s0[ok, 0].sum())) <= 0.02 * s0[ok, 0].sum()


# ---------------------------------------------------------------- golden fixtures

def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, ds, es, ls, _src = [f.strip() for f in line.split("|")]

        def num(tok):
            tok = tok.strip()
            neg = tok.startswith("-")
            t = tok[1:] if neg else tok
            if "sqrt" in t:
                a, b = t.split("sqrt") if not t.startswith("sqrt") else ("", t[4:])
                base = float(a.rstrip("+-")) if a else 0.0
                sgn = -1.0 if a.endswith("-") else 1.0
                v = base + sgn * math.sqrt(float(b))
            else:
                v = float(t)
            return -v if neg else v

        d = [num(x) for x in ds.split(",")]
        e = [num(x) for x in es.split(",")] if es else []
        lam = sorted(num(x) for x in ls.split(","))
        rows.append((name, d, e, lam))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: r[0])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_golden_closed_forms(oracle_mod, row, dt):
    name, d, e, lam_ref = row
    n = len(d)
    d = np.array([d], dtype=dt)
    e = np.array([e], dtype=dt).reshape(1, n - 1)
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    assert info[0] == 0
    tn = max(V.tnorm1(d, e)[0], 1.0)
    assert np.abs(lam[0].astype(np.float64) - np.array(lam_ref)).max() <= V.tol_of(dt, n) * tn
    assert V.band_residual(d, e, lam, Q)[0] <= V.tol_of(dt, n)
    assert V.orthogonality(Q)[0] <= V.tol_of(dt, n)


# ---------------------------------------------------------------- Toeplitz closed form

@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 12, 16, 31, 32, 64])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_toeplitz_closed_form(oracle_mod, n, dt, scheme):
    """tridiag(b; a; b): lambda_k = a + 2b cos(k pi/(n+1)) and eigenvectors
    sqrt(2/(n+1)) sin(j k pi/(n+1)) up to sign."""
    for a, b in ((2.0, -1.0), (0.3, 1.7), (-5.0, 0.25)):
        d, e = W.toeplitz_batch(n, a, b, 1, dt)
        lam, Q, info, _ = oracle_mod.steqr(d, e, True, scheme=scheme)
        assert info[0] == 0
        k = np.arange(1, n + 1)
        ref = np.sort(a + 2 * b * np.cos(k * np.pi / (n + 1)))
        tol = V.tol_of(dt, n)
        tn = V.tnorm1(d, e)[0]
        assert np.abs(lam[0] - ref).max() <= tol * tn
        # eigenvectors: the closed form is for the unsorted index k; match by value
        if n > 1 and b != 0:
            j = np.arange(1, n + 1)
            for kk in range(1, n + 1):
                val = a + 2 * b * math.cos(kk * math.pi / (n + 1))
                col = int(np.argmin(np.abs(lam[0] - val)))
                v = math.sqrt(2.0 / (n + 1)) * np.sin(j * kk * math.pi / (n + 1))
                q = Q[0, :, col].astype(np.float64)
                dist = min(np.abs(q - v).max(), np.abs(q + v).max())
                # eigenvalue gaps are >= ~|b| pi^2/(n+1)^2, so the vector error
                # is bounded by tol*||T|| / gap
                gap = abs(b) * (math.pi / (n + 1)) ** 2
                assert dist <= 4 * tol * tn / gap + 1e-12


# ---------------------------------------------------------------- configurations

SAMPLE = 256


@pytest.mark.parametrize("wname", list(W.WORKLOADS))
def test_workload_items_vs_sturm_and_invariants(oracle_mod, wname):
    """First items of every configuration: eigenvalues against long-double
    Sturm bisection (n <= 32 here), residual, orthogonality, trace and
    Frobenius invariants, for each item that converged."""
    w = W.WORKLOADS[wname]
    nb = 64 if w.n <= 32 else (16 if w.n <= 256 else 4)
    d, e = W.make_batch(w, nb)
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    ok = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    assert np.all(info[ok] == 0)
    tol = V.tol_of(d.dtype, w.n)
    dd, ee = d[ok], e[ok]
    ref = V.sturm_eigvals(dd, ee, iters=90 if w.n > 32 else 140).astype(np.float64)
    assert V.sorted_err(lam[ok], ref, dd, ee).max() <= tol
    assert V.band_residual(dd, ee, lam[ok], Q[ok]).max() <= tol
    assert V.orthogonality(Q[ok]).max() <= tol
    tn = V.tnorm1(dd, ee)
    l64 = lam[ok].astype(np.float64)
    d64, e64 = dd.astype(np.float64), ee.astype(np.float64)
    assert np.all(np.abs(l64.sum(1) - d64.sum(1)) <= w.n * tol * tn)
    fro = (d64 ** 2).sum(1) + 2 * (e64 ** 2).sum(1)
    assert np.all(np.abs((l64 ** 2).sum(1) - fro) <= 4 * w.n * tol * tn * tn)


@pytest.mark.parametrize("wname", ["c2_f32_n16", "c3_f64_n16", "c4_f64_n32", "c5_f64_n64"])
def test_workload_vs_numpy_eigvalsh(oracle_mod, wname):
    w = W.WORKLOADS[wname]
    d, e = W.make_batch(w, SAMPLE)
    lam, _, info, _ = oracle_mod.steqr(d, e, False)
    ok = np.isfinite(d).all(1) & np.isfinite(e).all(1)
    ref = np.linalg.eigvalsh(W.dense_from_bands(d[ok].astype(np.float64), e[ok].astype(np.float64)))
    assert V.sorted_err(lam[ok], ref, d[ok], e[ok]).max() <= V.tol_of(d.dtype, w.n)


def test_cross_precision_same_base(oracle_mod):
    """float32 and float64 items of the mixed configuration share their base
    matrices: their eigenvalues agree within the float32 tolerance."""
    w32, w64 = W.WORKLOADS["c4_f32_n32"], W.WORKLOADS["c4_f64_n32"]
    d32, e32 = W.make_batch(w32, 128)
    d64, e64 = W.make_batch(w64, 128)
    l32, _, i32, _ = oracle_mod.steqr(d32, e32, False)
    l64, _, i64, _ = oracle_mod.steqr(d64, e64, False)
    ok = (i32 == 0) & (i64 == 0)
    assert ok.sum() > 100
    assert V.sorted_err(l32[ok], l64[ok], d64[ok], e64[ok]).max() <= V.tol_of(np.float32, 32)


def test_jobz_n_matches_jobz_v_values(oracle_mod):
    d, e = W.make_batch(W.WORKLOADS["c2_f32_n16"], 128)
    lv, _, _, _ = oracle_mod.steqr(d, e, True)
    ln, _, _, _ = oracle_mod.steqr(d, e, False)
    assert np.array_equal(lv, ln)


def test_threads_bitwise_deterministic(oracle_mod):
    d, e = W.make_batch(W.WORKLOADS["c3_f64_n12"], 300)
    a = oracle_mod.steqr(d, e, True, threads=1)
    b = oracle_mod.steqr(d, e, True, threads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- edge items

@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [4, 16, 32])
def test_split_items_are_union_of_blocks(oracle_mod, dt, n):
    d, e = W.edge_batch(W.EDGE_SPLIT, n, 16, dt)
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    assert not info.any()
    cuts = [i for i in (n // 4 - 1, n // 2 - 1, 3 * n // 4 - 1) if 0 <= i < n - 1]
    for b in range(d.shape[0]):
        pieces = []
        lo = 0
        for c in cuts + [n - 1]:
            hi = c
            pieces.append(V.sturm_eigvals(d[b:b + 1, lo:hi + 1], e[b:b + 1, lo:hi])[0])
            lo = hi + 1
        ref = np.sort(np.concatenate(pieces)).astype(np.float64)
        assert V.sorted_err(lam[b:b + 1], ref[None], d[b:b + 1], e[b:b + 1])[0] <= V.tol_of(dt, n)
    # eigenvectors of a split matrix do not mix the blocks
    assert V.band_residual(d, e, lam, Q).max() <= V.tol_of(dt, n)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [1, 2, 5, 32, 64])
def test_zero_items_exact(oracle_mod, dt, n):
    d = np.zeros((3, n), dt)
    e = np.zeros((3, n - 1), dt)
    lam, Q, info, st = oracle_mod.steqr(d, e, True)
    assert not info.any()
    assert np.all(lam == 0)
    assert np.array_equal(Q, np.broadcast_to(np.eye(n, dtype=dt), Q.shape))
    assert not st.any()


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_graded_items_normwise(oracle_mod, dt):
    n = 32
    d, e = W.edge_batch(W.EDGE_GRADED, n, 24, dt)
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    assert not info.any()
    ref = V.sturm_eigvals(d, e).astype(np.float64)
    assert V.sorted_err(lam, ref, d, e).max() <= V.tol_of(dt, n)
    assert V.band_residual(d, e, lam, Q).max() <= V.tol_of(dt, n)
    assert V.orthogonality(Q).max() <= V.tol_of(dt, n)


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_scaled_items_against_twins(oracle_mod, dt):
    n = 32
    d, e = W.edge_batch(W.EDGE_SCALED, n, 24, np.float64)
    # item b of edge_batch is scaled by 1e18 (b even) or 1e-18 (b odd)
    f = np.where(np.arange(24) % 2 == 0, 1e18, 1e-18)
    base_d, base_e = d / f[:, None], e / f[:, None]
    lam, Q, info, _ = oracle_mod.steqr(d.astype(dt), e.astype(dt), True)
    bl, _, binfo, _ = oracle_mod.steqr(base_d.astype(dt), base_e.astype(dt), False)
    assert not info.any() and not binfo.any()
    err = V.sorted_err(lam.astype(np.float64) / f[:, None], bl, base_d, base_e)
    assert err.max() <= V.tol_of(dt, n)
    assert V.orthogonality(Q).max() <= V.tol_of(dt, n)


@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
@pytest.mark.parametrize("n", [3, 16, 32])
def test_nan_items_fail_with_budget(oracle_mod, dt, n, scheme):
    """A NaN never passes the deflation test, so the block holding it burns
    the whole 30n sweep budget: info > 0, the solve terminates, and the NaN
    spreads over that block only."""
    d, e = W.edge_batch(W.EDGE_NAN, n, 12, dt)
    lam, Q, info, st = oracle_mod.steqr(d, e, True, scheme=scheme)
    assert np.all(info > 0)
    assert np.all(st[:, 0] == 30 * n)
    # one block (random e has no zeros): every eigenvalue slot is NaN,
    # every off-diagonal nonzero
    assert np.all(np.isnan(lam))
    assert np.all(info == n - 1)


@pytest.mark.parametrize("scheme", [0, 1], ids=["exp", "pg"])
def test_nan_confined_to_its_block(oracle_mod, scheme):
    n = 12
    d, e = W.random_batch(n, 4, np.float64, salt=3)
    e[:, 5] = 0.0  # blocks [0,5] and [6,11]
    d[:, 8] = np.nan  # NaN in the second block
    lam, _, info, _ = oracle_mod.steqr(d, e, False, scheme=scheme)
    assert np.all(info == 5)  # e_6..e_10 of the NaN block stay nonzero
    assert np.all(np.isfinite(lam[:, :6])) and np.all(np.isnan(lam[:, 6:]))
    # the first block converged to its own eigenvalues (unsorted output)
    ref = V.sturm_eigvals(d[:, :6], e[:, :5]).astype(np.float64)
    assert V.sorted_err(lam[:, :6], ref, d[:, :6], e[:, :5]).max() <= V.tol_of(np.float64, 6)
    # a NaN before the block: the earlier blocks converge, later ones untouched
    d2, e2 = W.random_batch(n, 4, np.float64, salt=4)
    e2[:, 5] = 0.0
    d2[:, 2] = np.nan
    lam2, _, info2, _ = oracle_mod.steqr(d2, e2, False, scheme=scheme)
    assert np.all(info2 == 5 + 5)
    assert np.all(np.isnan(lam2[:, :6]))
    assert np.array_equal(lam2[:, 6:], d2[:, 6:])


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["f32", "f64"])
def test_sweep_cap_forces_info(oracle_mod, dt):
    d, e = W.random_batch(16, 20, dt, salt=8)
    lam, _, info, st = oracle_mod.steqr(d, e, False, max_sweeps_per_n=0)
    assert np.all(info > 0) and not st[:, 0].any()
    # no sweep was allowed and random items have no 2x2 tail: the values
    # come back exactly as given (the block reversal is undone exactly)
    assert np.array_equal(lam, d)
    lam1, _, info1, st1 = oracle_mod.steqr(d, e, False, max_sweeps_per_n=1)
    assert np.all(st1[:, 0] <= 16)
    lam30, _, info30, _ = oracle_mod.steqr(d, e, False)
    assert not info30.any()


def test_unsorted_output_is_a_permutation(oracle_mod):
    d, e = W.random_batch(9, 30, np.float64, salt=2)
    ls, Qs, _, _ = oracle_mod.steqr(d, e, True, sort=True)
    lu, Qu, _, _ = oracle_mod.steqr(d, e, True, sort=False)
    assert np.array_equal(np.sort(lu, axis=1), ls)
    assert V.band_residual(d, e, lu, Qu).max() <= V.tol_of(np.float64, 9)


def test_n1_and_n2_special_cases(oracle_mod):
    d = np.array([[4.0], [-2.5]])
    e = np.zeros((2, 0))
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    assert np.array_equal(lam, d) and np.all(Q == 1.0) and not info.any()
    d = np.array([[1.0, 3.0]])
    e = np.array([[2.0]])
    lam, Q, info, _ = oracle_mod.steqr(d, e, True)
    ref = [2 - math.sqrt(5), 2 + math.sqrt(5)]
    assert np.abs(lam[0] - ref).max() <= 1e-15
