"""Core pins of the CPU oracle against mathematics independent of it.

Each pin returns a list of failure strings (empty = pinned). They are run
by tests/test_oracle_pins.py on the real oracle, and on deliberately broken
copies of the oracle source (tests/test_oracle_mutants.py) to show that a
plausible mistake anywhere in the oracle fails at least one of them.

What each pin checks, and why it is independent of the oracle's own code:
  lartg      the defining relations of the Givens rotation on the pages
             (G^T (f,g) = (r,0), c^2 + s^2 = 1) and its stated special case
             g = 0 -> (1, 0, f), plus overflow-free behaviour at 1e+-30 in f32;
  shift      the LAPACK-form shift equals the closed-form 2x2 eigenvalue
             nearest the endpoint (quadratic formula, long double);
  sym2x2     the analytic 2x2 solve against the same closed form and the
             diagonalisation J^T B J = diag;
  sweep      one implicit sweep against an explicit shifted QR step
             T - mu I = QR, T' = RQ + mu I (numpy QR in float64): by the
             implicit-Q theorem the two agree up to the signs of e; and the
             accumulated rotations reproduce T' = Q^T T Q;
  solve      whole solves against Sturm-count bisection in long double, the
             residual and orthogonality bounds, the trace and Frobenius
             invariants, the Kac-Sylvester-Clement matrix (integer spectrum),
             and the scaling identity lambda(1e18 T) = 1e18 lambda(T);
  back-transform  with a basis Z on entry the result is Z times the
             rotations: Z = I reproduces the plain solve bit for bit; for an
             orthogonal Z the columns are eigenvectors of the dense
             A = Z T Z^T (numpy matmul in float64); for a general Z the
             result matches the matmul Z Q; a solve that performs no
             rotation returns Z unchanged;
  larfg      the reflector's defining relations H x = (beta, 0..0), H
             orthogonal, |beta| = ||x||, sign(beta) = -sign(alpha), in long
             double, and the stated special case x_1..m = 0 -> H = I;
  sytrd      A = Q T Q^T and Q^T Q = I by numpy matmul in float64, the
             spectrum of T (long-double Sturm bisection) against numpy's
             eigvalsh of A, d_0 = a_00 and |e_0| = ||a_{1:,0}|| exactly as
             the first step fixes them, a tridiagonal A returned unchanged
             with Q = I, and the strict upper triangle never read;
  syev       eigenvalues against numpy's eigvalsh, the dense residual and
             orthogonality bounds, a tridiagonal A giving the tridiagonal
             solve bit for bit, and a diagonal A its sorted diagonal with a
             permutation for Q;
  stebz      the Sturm count against numpy's eigvalsh (the number of
             eigenvalues below x, at points away from them), whole solves
             against eigvalsh, the Clement and Toeplitz closed forms and the
             QR solve, ascending output, exact power-of-two scaling
             lambda(2^j T) = 2^j lambda(T), a diagonal T, T = 0 and NaN.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

import validate as V
import workloads as W


def _fail(out: List[str], cond: bool, msg: str) -> None:
    if not cond:
        out.append(msg)


def pin_lartg(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    rng = np.random.default_rng(7)
    for dt in (np.float32, np.float64):
        eps = V.eps_of(dt)
        pairs = list(zip(rng.standard_normal(200), rng.standard_normal(200)))
        pairs += [(3.0, 4.0), (-3.0, 4.0), (3.0, -4.0), (-3.0, -4.0), (1e-3, 5.0),
                  (7.0, 1e-6)]
        if dt == np.float32:
            pairs += [(1e30, 3e30), (-2e30, 1e30), (1e-30, -3e-30), (4e-30, 1e-30),
                      (1e30, 1e-30)]
        else:
            pairs += [(1e300, 3e300), (1e-300, -2e-300)]
        for f, g in pairs:
            f = float(dt(f))
            g = float(dt(g))
            c, s, r = oracle.lartg(f, g, dt, libpath)
            if not all(map(math.isfinite, (c, s, r))):
                out.append("lartg non-finite for (%g,%g)" % (f, g))
                continue
            scale = max(abs(f), abs(g))
            fl, gl, cl, sl, rl = (np.longdouble(v) for v in (f, g, c, s, r))
            _fail(out, abs(cl * fl + sl * gl - rl) <= 4 * eps * scale,
                  "lartg c f + s g != r at (%g,%g)" % (f, g))
            _fail(out, abs(-sl * fl + cl * gl) <= 4 * eps * scale,
                  "lartg -s f + c g != 0 at (%g,%g)" % (f, g))
            _fail(out, abs(cl * cl + sl * sl - 1) <= 4 * eps,
                  "lartg c^2+s^2 != 1 at (%g,%g)" % (f, g))
            _fail(out, c >= 0 and (r == 0 or math.copysign(1, r) == math.copysign(1, f)),
                  "lartg sign convention (c >= 0, sign r = sign f) at (%g,%g)" % (f, g))
        for f in (2.5, -1.0, 0.0):
            c, s, r = oracle.lartg(f, 0.0, dt, libpath)
            _fail(out, (c, s, r) == (1.0, 0.0, f), "lartg(f, 0) != (1, 0, f)")
        c, s, r = oracle.lartg(0.0, -2.0, dt, libpath)
        _fail(out, (c, s, r) == (0.0, -1.0, 2.0), "lartg(0, g) != (0, sign g, |g|)")
    return out


def _closest_eig(d1, d2, e1):
    """Eigenvalue of [[d2, e1], [e1, d1]] nearest d1, by the quadratic formula
    of the algorithm page's shift section, in long double."""
    a, c, b = np.longdouble(d2), np.longdouble(d1), np.longdouble(e1)
    mid = (a + c) / 2
    rad = np.sqrt(((a - c) / 2) ** 2 + b * b)
    lp, lm = mid + rad, mid - rad
    return lp if abs(lp - c) < abs(lm - c) else lm


def pin_shift(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    rng = np.random.default_rng(11)
    for dt in (np.float32, np.float64):
        eps = V.eps_of(dt)
        trip = [tuple(map(float, rng.standard_normal(3))) for _ in range(300)]
        trip += [(0.0, 2.0, 1.0), (2.0, 0.0, 1.0), (1.0, 1.0, 1e-3), (5.0, -5.0, 1e-2)]
        for d1, d2, e1 in trip:
            d1, d2, e1 = (float(dt(v)) for v in (d1, d2, e1))
            if e1 == 0:
                continue
            ref = _closest_eig(d1, d2, e1)
            scale = abs(d1) + abs(d2) + abs(e1)
            # when both eigenvalues are (nearly) equally close to d1 either
            # one is the nearest up to rounding
            a, c, b = np.longdouble(d2), np.longdouble(d1), np.longdouble(e1)
            rad = np.sqrt(((a - c) / 2) ** 2 + b * b)
            lp, lm = (a + c) / 2 + rad, (a + c) / 2 - rad
            tie = abs(abs(lp - c) - abs(lm - c)) <= 8 * eps * scale
            for closed in (False, True):
                mu = np.longdouble(oracle.shift(d1, d2, e1, dt, libpath, closed=closed))
                ok = abs(mu - ref) <= 8 * eps * scale or \
                    (tie and min(abs(mu - lp), abs(mu - lm)) <= 8 * eps * scale)
                _fail(out, ok, "shift(%g,%g,%g, closed=%s)=%r, closed form %r"
                      % (d1, d2, e1, closed, float(mu), float(ref)))
    return out


def pin_sym2x2(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    rng = np.random.default_rng(13)
    for dt in (np.float32, np.float64):
        eps = V.eps_of(dt)
        trip = [tuple(map(float, rng.standard_normal(3))) for _ in range(300)]
        trip += [(1.0, 1.0, 1.0), (2.0, 0.0, 2.0), (0.0, 1e-20, 1.0), (3.0, 4.0, -3.0)]
        for a, b, c in trip:
            a, b, c = (float(dt(v)) for v in (a, b, c))
            rt1, rt2, cs, sn = oracle.sym2x2(a, b, c, dt, libpath)
            A, B, C = (np.longdouble(v) for v in (a, b, c))
            mid = (A + C) / 2
            rad = np.sqrt(((A - C) / 2) ** 2 + B * B)
            got = sorted([np.longdouble(rt1), np.longdouble(rt2)])
            scale = abs(a) + abs(b) + abs(c)
            _fail(out, abs(got[0] - (mid - rad)) <= 8 * eps * scale and
                  abs(got[1] - (mid + rad)) <= 8 * eps * scale,
                  "sym2x2 eigenvalues (%g,%g,%g)" % (a, b, c))
            J = np.array([[cs, sn], [-sn, cs]], dtype=np.longdouble)
            Bm = np.array([[A, B], [B, C]], dtype=np.longdouble)
            D = J.T @ Bm @ J
            _fail(out, abs(D[0, 1]) <= 8 * eps * scale and
                  abs(D[0, 0] - np.longdouble(rt1)) <= 8 * eps * scale and
                  abs(D[1, 1] - np.longdouble(rt2)) <= 8 * eps * scale,
                  "sym2x2 rotation does not diagonalise (%g,%g,%g)" % (a, b, c))
            _fail(out, abs(np.longdouble(cs) ** 2 + np.longdouble(sn) ** 2 - 1) <= 4 * eps,
                  "sym2x2 rotation not orthogonal")
    return out


def pin_sweep(oracle, libpath: Optional[str] = None, scheme: int = 0) -> List[str]:
    """One implicit sweep (EXP form, scheme 0, or PG form, scheme 1) against
    an explicit shifted QR step."""
    out: List[str] = []
    rng = np.random.default_rng(17)
    n = 10
    for trial in range(20):
        d = rng.standard_normal(n)
        e = rng.standard_normal(n - 1)
        s, m = (0, n - 1) if trial % 2 == 0 else (2, 7)
        mu = float(rng.standard_normal())
        d1, e1 = d.copy(), e.copy()
        Qs = np.eye(n)
        rots = oracle.sweep(d1, e1, Qs, s, m, mu, libpath, scheme=scheme)
        _fail(out, rots == m - s, "sweep rotation count %d != %d" % (rots, m - s))
        T = W.dense_from_bands(d[None], e[None])[0]
        # explicit step on the unreduced sub-block [s, m]
        blk = T[s:m + 1, s:m + 1]
        Qe, Re = np.linalg.qr(blk - mu * np.eye(m - s + 1))
        T1 = Re @ Qe + mu * np.eye(m - s + 1)
        dref = np.diag(T1)
        eref = np.diag(T1, 1)
        scale = np.abs(blk).sum(axis=0).max()
        tol = 1e-12 * scale
        _fail(out, np.abs(d1[s:m + 1] - dref).max() <= tol,
              "sweep diagonal differs from explicit QR step (trial %d)" % trial)
        _fail(out, np.abs(np.abs(e1[s:m]) - np.abs(eref)).max() <= tol,
              "sweep off-diagonal differs from explicit QR step (trial %d)" % trial)
        # untouched parts stay untouched
        _fail(out, np.array_equal(d1[:s], d[:s]) and np.array_equal(d1[m + 1:], d[m + 1:]),
              "sweep touched d outside [s, m]")
        # accumulated rotations reproduce the new tridiagonal
        T1full = Qs.T @ T @ Qs
        T1b = W.dense_from_bands(d1[None], e1[None])[0]
        if s > 0:
            # couplings to the rest of the matrix are outside the sweep; keep them
            T1b[s - 1, s] = T1full[s - 1, s]
            T1b[s, s - 1] = T1full[s, s - 1]
        if m < n - 1:
            T1b[m, m + 1] = T1full[m, m + 1]
            T1b[m + 1, m] = T1full[m + 1, m]
        _fail(out, np.abs(T1full[s:m + 1, s:m + 1] - T1b[s:m + 1, s:m + 1]).max() <= tol,
              "accumulated Q does not reproduce the swept block (trial %d)" % trial)
        # invariants: trace and Frobenius norm of the block
        _fail(out, abs(d1[s:m + 1].sum() - d[s:m + 1].sum()) <= tol,
              "sweep trace not preserved")
        fro0 = (d[s:m + 1] ** 2).sum() + 2 * (e[s:m] ** 2).sum()
        fro1 = (d1[s:m + 1] ** 2).sum() + 2 * (e1[s:m] ** 2).sum()
        _fail(out, abs(fro1 - fro0) <= 1e-12 * fro0, "sweep Frobenius norm not preserved")
    # a sweep with an exact eigenvalue of the trailing 2x2 as shift on a
    # 2x2 block deflates it
    d = np.array([1.0, 3.0])
    e = np.array([0.5])
    mu = float(_closest_eig(3.0, 1.0, 0.5))
    oracle.sweep(d, e, None, 0, 1, mu, libpath, scheme=scheme)
    _fail(out, abs(e[0]) <= 1e-14, "exact shift does not deflate a 2x2 (e=%g)" % e[0])
    _fail(out, abs(d[1] - mu) <= 1e-14, "exact shift: d_m != mu")
    return out


def clement(n: int):
    """Symmetric Kac-Sylvester-Clement matrix: zero diagonal, e_k =
    sqrt(k (n-k)); its eigenvalues are -(n-1), -(n-3), ..., n-1."""
    d = np.zeros((1, n))
    k = np.arange(1, n)
    e = np.sqrt(k * (n - k)).reshape(1, -1).astype(np.float64)
    lam = np.arange(-(n - 1), n, 2, dtype=np.float64)
    return d, e, lam


def pin_solve(oracle, libpath: Optional[str] = None, quick: bool = False,
              scheme: int = 0, shift: int = 0) -> List[str]:
    out: List[str] = []
    sizes = (3, 8, 13) if quick else (1, 2, 3, 5, 8, 13, 16, 100)
    for dt in (np.float32, np.float64):
        for n in sizes:
            d, e = W.random_batch(n, 16 if quick else 48, dt, salt=5)
            lam, Q, info, _ = oracle.steqr(d, e, True, libpath=libpath, scheme=scheme, shift=shift)
            _fail(out, not info.any(), "solve info != 0 (%s n=%d)" % (dt.__name__, n))
            tol = V.tol_of(dt, n)
            ref = V.sturm_eigvals(d, e)
            err = V.sorted_err(lam, ref.astype(np.float64), d, e)
            _fail(out, err.max() <= tol, "solve vs Sturm %s n=%d: %g > %g"
                  % (dt.__name__, n, err.max(), tol))
            _fail(out, np.all(np.diff(lam, axis=1) >= 0), "solve output not ascending")
            res = V.band_residual(d, e, lam, Q)
            _fail(out, res.max() <= tol, "solve residual %s n=%d: %g" % (dt.__name__, n, res.max()))
            orth = V.orthogonality(Q)
            _fail(out, orth.max() <= tol, "solve orthogonality %s n=%d: %g"
                  % (dt.__name__, n, orth.max()))
            lam64 = lam.astype(np.float64)
            dd, ee = d.astype(np.float64), e.astype(np.float64)
            tn = V.tnorm1(d, e)
            tr = np.abs(lam64.sum(1) - dd.sum(1))
            _fail(out, np.all(tr <= n * tol * tn), "trace invariant %s n=%d" % (dt.__name__, n))
            fro = (dd ** 2).sum(1) + 2 * (ee ** 2).sum(1)
            _fail(out, np.all(np.abs((lam64 ** 2).sum(1) - fro) <= 4 * n * tol * tn * tn),
                  "Frobenius invariant %s n=%d" % (dt.__name__, n))
    for n in ((8, 16) if quick else (4, 8, 16, 32, 64, 128)):
        d, e, ref = clement(n)
        for dt in (np.float32, np.float64):
            lam, Q, info, _ = oracle.steqr(d.astype(dt), e.astype(dt), True, libpath=libpath, scheme=scheme, shift=shift)
            tol = V.tol_of(dt, n)
            err = np.abs(lam[0].astype(np.float64) - ref).max() / V.tnorm1(d, e)[0]
            _fail(out, info[0] == 0 and err <= tol, "Clement n=%d %s: %g" % (n, dt.__name__, err))
    # scaling identity lambda(f T) = f lambda(T). float32: 1e18 straddles
    # ssfmax = 2^63/3, 1e19 is above it, 1e-18 below ssfmin = 2^-15;
    # float64: 1e200 above ssfmax = 2^511/3, 1e-200 below ssfmin = 2^-405.
    n = 12
    d, e = W.random_batch(n, 32, np.float64, salt=9)
    for dt, factors in ((np.float32, (1e18, 1e19, 1e-18)), (np.float64, (1e200, 1e-200))):
        base_l, _, _, _ = oracle.steqr(d.astype(dt), e.astype(dt), False, libpath=libpath, scheme=scheme, shift=shift)
        for f in factors:
            lam, Q, info, _ = oracle.steqr((d * f).astype(dt), (e * f).astype(dt), True,
                                           libpath=libpath, scheme=scheme, shift=shift)
            err = V.sorted_err(lam.astype(np.float64) / f, base_l, d, e)
            _fail(out, not info.any() and err.max() <= V.tol_of(dt, n),
                  "scaling identity %s at %g: %g" % (dt.__name__, f, err.max()))
            orth = V.orthogonality(Q).max()
            _fail(out, orth <= V.tol_of(dt, n), "scaled orthogonality %s at %g" % (dt.__name__, f))
    return out


def _graded(n: int, batch: int, dt, small_end_top: bool):
    """Graded items of the workload recipe (d_i = 10^(-i/2), coupling
    z_i sqrt(d_i d_{i+1})): the small end is the bottom; reversed, the top."""
    d, e = W.edge_batch(W.EDGE_NAMES.index("graded"), n, batch, np.float64)
    if small_end_top:
        d, e = d[:, ::-1].copy(), e[:, ::-1].copy()
    return d.astype(dt), e.astype(dt)


def pin_direction(oracle, libpath: Optional[str] = None, quick: bool = False,
                  scheme: int = 0, shift: int = 0) -> List[str]:
    """The choice of the converging end ("STEQR: the CTA tridiagonal solver",
    micro-structure list, QL versus QR; the steqr algorithm page, QR/QL
    paragraph): a graded block must converge its small end first. By the CTA
    page the opposite choice roughly doubled the number of steps and gave
    worse relative errors for graded matrices. Pinned on graded items with the
    small end at the bottom and, reversed, at the top (a rule that always or
    never reverses fails one of the two):
      * implicit sweeps per eigenvalue, averaged over the batch, at most 1.5
        (the right rule takes 1.0-1.3 at orders 8-32; the opposite one 1.6-2.4);
      * every eigenvalue within a relative error of 2^-10 (float) or 2^-30
        (double) of its long-double Sturm value (the right rule stays below
        5e-4 / 4e-13; the opposite one loses every digit of the small
        eigenvalues at order 32);
      * the normwise residual and orthogonality bounds still hold.
    """
    out: List[str] = []
    for dt, rel_tol in ((np.float32, 2.0 ** -10), (np.float64, 2.0 ** -30)):
        for n in ((16, 32) if quick else (8, 16, 32)):
            for top in (False, True):
                d, e = _graded(n, 16 if quick else 64, dt, top)
                lam, Q, info, st = oracle.steqr(d, e, True, libpath=libpath,
                                                scheme=scheme, shift=shift)
                tag = "%s n=%d small end %s" % (dt.__name__, n, "top" if top else "bottom")
                _fail(out, not info.any(), "graded solve info != 0 (%s)" % tag)
                per_eig = st[:, 0].mean() / n
                _fail(out, per_eig <= 1.5, "graded sweeps per eigenvalue %.2f > 1.5 (%s)"
                      % (per_eig, tag))
                ref = np.sort(V.sturm_eigvals(d, e).astype(np.float64), axis=1)
                got = np.sort(lam.astype(np.float64), axis=1)
                rel = np.abs(got - ref) / np.abs(ref)
                _fail(out, rel.max() <= rel_tol, "graded relative error %.3g > %.3g (%s)"
                      % (rel.max(), rel_tol, tag))
                tol = V.tol_of(dt, n)
                _fail(out, V.band_residual(d, e, lam, Q).max() <= tol
                      and V.orthogonality(Q).max() <= tol, "graded residual (%s)" % tag)
    return out


def pin_block2(oracle, libpath: Optional[str] = None, quick: bool = False,
               scheme: int = 0, shift: int = 0) -> List[str]:
    """A block of order 2 is solved in closed form (steqr algorithm page,
    2x2 block paragraph), not by implicit sweeps: order-2 items and items
    split into 2x2 blocks by exact zeros take no sweep at all (so they also
    converge with a sweep budget of zero), count one analytic solve per
    block, and return the closed-form eigenvalues (a+c)/2 +- sqrt(((a-c)/2)^2
    + b^2) of each block (long double) within 8 eps ||T||, with eigenvectors
    meeting the residual and orthogonality bounds."""
    out: List[str] = []
    for dt in (np.float32, np.float64):
        eps = V.eps_of(dt)
        for n, zeros in ((2, ()), (8, (1, 3, 5)), (12, (1, 3, 5, 7, 9))):
            d, e = W.random_batch(n, 24, dt, salt=31)
            for z in zeros:
                e[:, z] = 0
            blocks = n // 2
            tn = V.tnorm1(d, e)
            A = d[:, 0::2].astype(np.longdouble)
            C = d[:, 1::2].astype(np.longdouble)
            B = np.concatenate([e, np.zeros((e.shape[0], 1), dt)], 1)[:, 0::2].astype(np.longdouble)
            mid, rad = (A + C) / 2, np.sqrt(((A - C) / 2) ** 2 + B * B)
            ref = np.sort(np.concatenate([mid - rad, mid + rad], 1).astype(np.float64), axis=1)
            for budget in (30, 0):
                lam, Q, info, st = oracle.steqr(d, e, True, max_sweeps_per_n=budget,
                                                libpath=libpath, scheme=scheme, shift=shift)
                tag = "%s n=%d budget %d" % (dt.__name__, n, budget)
                _fail(out, not info.any(), "2x2 blocks did not converge (%s)" % tag)
                _fail(out, np.all(st[:, 0] == 0) and np.all(st[:, 1] == 0),
                      "2x2 blocks took implicit sweeps (%s)" % tag)
                _fail(out, np.all(st[:, 2] == blocks), "2x2 blocks: %s analytic solves, "
                      "expected %d (%s)" % (np.unique(st[:, 2]), blocks, tag))
                err = np.abs(np.sort(lam.astype(np.float64), axis=1) - ref).max(1) / tn
                _fail(out, err.max() <= 8 * eps, "2x2 blocks against the closed form: %g (%s)"
                      % (err.max(), tag))
                tol = V.tol_of(dt, n)
                _fail(out, V.band_residual(d, e, lam, Q).max() <= tol
                      and V.orthogonality(Q).max() <= tol, "2x2 blocks residual (%s)" % tag)
    return out


def pin_large_orders(oracle, libpath: Optional[str] = None, scheme: int = 0,
                     shift: int = 0) -> List[str]:
    """Orders 129..512 (beyond the largest sub-group-width kernels): random
    items against long-double Sturm bisection with the residual and
    orthogonality bounds, the Kac-Sylvester-Clement integer spectrum and the
    Toeplitz closed form a + 2b cos(k pi/(n+1)) at orders 256 and 512."""
    out: List[str] = []
    kw = dict(libpath=libpath, scheme=scheme, shift=shift)
    for dt in (np.float32, np.float64):
        for n in (129, 200, 256, 300, 512):
            d, e = W.random_batch(n, 4 if n <= 256 else 2, dt, salt=77)
            lam, Q, info, _ = oracle.steqr(d, e, True, **kw)
            tol = V.tol_of(dt, n)
            ref = V.sturm_eigvals(d, e).astype(np.float64)
            err = V.sorted_err(lam, ref, d, e).max()
            _fail(out, not info.any() and err <= tol, "order %d %s vs Sturm: %g" % (n, dt.__name__, err))
            _fail(out, V.band_residual(d, e, lam, Q).max() <= tol
                  and V.orthogonality(Q).max() <= tol, "order %d %s residual" % (n, dt.__name__))
        for n in (256, 512):
            cd, ce, cref = clement(n)
            lam, _, info, _ = oracle.steqr(cd.astype(dt), ce.astype(dt), False, **kw)
            err = np.abs(lam[0].astype(np.float64) - cref).max() / V.tnorm1(cd, ce)[0]
            _fail(out, info[0] == 0 and err <= V.tol_of(dt, n),
                  "Clement %d %s: %g" % (n, dt.__name__, err))
            a, b = 0.5, -1.25
            td = np.full((1, n), a)
            te = np.full((1, n - 1), b)
            k = np.arange(1, n + 1)
            tref = np.sort(a + 2 * b * np.cos(k * np.pi / (n + 1)))
            lam, _, info, _ = oracle.steqr(td.astype(dt), te.astype(dt), False, **kw)
            err = np.abs(lam[0].astype(np.float64) - tref).max() / V.tnorm1(td, te)[0]
            _fail(out, info[0] == 0 and err <= V.tol_of(dt, n),
                  "Toeplitz %d %s: %g" % (n, dt.__name__, err))
    return out


def pin_back_transform(oracle, libpath: Optional[str] = None, quick: bool = False,
                       scheme: int = 0, shift: int = 0) -> List[str]:
    """Eigenvector accumulation with a basis on entry (algorithm page,
    eigenvector paragraph: the rotations right-multiply the caller's basis
    instead of the identity)."""
    out: List[str] = []
    kw = dict(libpath=libpath, scheme=scheme, shift=shift)
    for dt in (np.float32, np.float64):
        for n in ((1, 5, 16) if quick else (1, 2, 3, 7, 16, 33)):
            batch = 12
            d, e = W.random_batch(n, batch, dt, salt=21)
            l0, Q0, i0, _ = oracle.steqr(d, e, True, **kw)
            ident = np.ascontiguousarray(np.broadcast_to(np.eye(n, dtype=dt), (batch, n, n)))
            l1, Q1, i1, _ = oracle.steqr(d, e, True, Z=ident, **kw)
            _fail(out, np.array_equal(l1, l0) and np.array_equal(Q1, Q0)
                  and np.array_equal(i1, i0), "Z = I differs from Q <- I (%s n=%d)"
                  % (dt.__name__, n))
            tol = V.tol_of(dt, n)
            Z = W.random_basis(n, batch, dt, salt=3)
            Zin = Z.copy()
            l2, Q2, i2, _ = oracle.steqr(d, e, True, Z=Z, **kw)
            _fail(out, np.array_equal(Z, Zin), "the basis was modified")
            _fail(out, np.array_equal(l2, l0) and np.array_equal(i2, i0),
                  "eigenvalues depend on the basis (%s n=%d)" % (dt.__name__, n))
            Z64 = Z.astype(np.float64)
            A = np.matmul(np.matmul(Z64, W.dense_from_bands(d.astype(np.float64),
                                                            e.astype(np.float64))),
                          np.swapaxes(Z64, 1, 2))
            res = V.dense_residual(A, l2, Q2)
            _fail(out, res.max() <= tol, "dense residual with orthogonal Z %s n=%d: %g"
                  % (dt.__name__, n, res.max()))
            _fail(out, V.orthogonality(Q2).max() <= tol,
                  "orthogonality with orthogonal Z %s n=%d" % (dt.__name__, n))
            G = W.random_basis(n, batch, dt, salt=4, orthogonal=False)
            _, Q3, _, _ = oracle.steqr(d, e, True, Z=G, **kw)
            ref = np.matmul(G.astype(np.float64), Q0.astype(np.float64))
            rowerr = np.sqrt(((Q3.astype(np.float64) - ref) ** 2).sum(-1))
            rown = np.sqrt((G.astype(np.float64) ** 2).sum(-1))
            _fail(out, np.all(rowerr <= tol * rown), "general Z: not Z times the rotations "
                  "(%s n=%d): %g" % (dt.__name__, n, (rowerr / rown).max()))
        # a zero sweep budget on unreduced blocks of order >= 3 stops before
        # the first rotation: Q must be the basis itself
        n = 6
        d, e = W.random_batch(n, 4, dt, salt=22)
        G = W.random_basis(n, 4, dt, salt=5, orthogonal=False)
        _, Q4, i4, _ = oracle.steqr(d, e, True, max_sweeps_per_n=0, Z=G, **kw)
        _fail(out, np.all(i4 > 0) and np.array_equal(Q4, G),
              "failed solve with no rotation changed the basis (%s)" % dt.__name__)
    return out


def pin_larfg(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    g = np.random.default_rng(31)
    for dt in (np.float32, np.float64):
        eps = V.eps_of(dt)
        for m in (1, 2, 5, 15):
            for trial in range(6):
                x = g.standard_normal(m + 1).astype(dt)
                if trial == 1:
                    x[0] = -abs(x[0])
                if trial == 2:
                    x *= dt(1e15) if dt == np.float32 else 1e150   # no overflow
                if trial == 3:
                    x[0] = 0
                beta, tau, v = oracle.larfg(x[0], x[1:], libpath=libpath)
                X = x.astype(np.longdouble)
                u = np.concatenate([[1], v.astype(np.longdouble)])
                Hx = X - np.longdouble(tau) * u * (u @ X)
                xn = np.sqrt((X ** 2).sum())
                _fail(out, np.abs(Hx[1:]).max() <= 8 * m * eps * xn and
                      abs(Hx[0] - np.longdouble(beta)) <= 8 * m * eps * xn,
                      "larfg H x != (beta, 0) (%s m=%d trial %d)" % (dt.__name__, m, trial))
                _fail(out, abs(abs(np.longdouble(beta)) - xn) <= 4 * eps * xn,
                      "larfg |beta| != ||x|| (%s m=%d)" % (dt.__name__, m))
                # H orthogonal <=> tau^2 ||u||^2 = 2 tau
                t = np.longdouble(tau)
                _fail(out, abs(t * t * (u @ u) - 2 * t) <= 16 * m * eps,
                      "larfg H not orthogonal (%s m=%d)" % (dt.__name__, m))
                _fail(out, (beta < 0) == (x[0] >= 0) or np.abs(x[1:]).max() == 0,
                      "larfg sign of beta (%s m=%d)" % (dt.__name__, m))
        for alpha in (2.5, -2.5, 0.0):
            beta, tau, v = oracle.larfg(alpha, np.zeros(3, dtype=dt), libpath=libpath)
            _fail(out, tau == 0 and beta == alpha and np.all(v == 0),
                  "larfg x = 0 is not H = I (%s)" % dt.__name__)
    return out


def _sym_from_lower(A) -> np.ndarray:
    L = np.tril(np.asarray(A, dtype=np.float64))
    return L + np.swapaxes(np.tril(L, -1), 1, 2)


def pin_sytrd(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    for dt in (np.float32, np.float64):
        for n in (1, 2, 3, 4, 7, 16, 32):
            A = W.random_symmetric(n, 10, dt, salt=51)
            d, e, Q = oracle.sytrd(A, libpath=libpath)
            tol = V.tol_of(dt, n)
            As = _sym_from_lower(A)
            an = np.abs(As).sum(1).max(1)
            T = W.dense_from_bands(d.astype(np.float64), e.astype(np.float64))
            Q64 = Q.astype(np.float64)
            rec = np.abs(Q64 @ T @ np.swapaxes(Q64, 1, 2) - As).sum(1).max(1)
            _fail(out, np.all(rec <= tol * an), "sytrd A != Q T Q^T (%s n=%d): %g"
                  % (dt.__name__, n, (rec / an).max()))
            _fail(out, V.orthogonality(Q).max() <= tol, "sytrd Q not orthogonal (%s n=%d)"
                  % (dt.__name__, n))
            ref = np.linalg.eigvalsh(As)
            lam = V.sturm_eigvals(d, e).astype(np.float64)
            _fail(out, np.all(np.abs(lam - ref).max(1) <= tol * an),
                  "sytrd spectrum of T != eigvalsh(A) (%s n=%d)" % (dt.__name__, n))
            _fail(out, np.array_equal(d[:, 0], A[:, 0, 0]), "sytrd d_0 != a_00")
            if n > 1:
                cn = np.sqrt((As[:, 1:, 0] ** 2).sum(1))
                _fail(out, np.all(np.abs(np.abs(e[:, 0]) - cn) <= 4 * n * V.eps_of(dt) * cn),
                      "sytrd |e_0| != ||a_{1:,0}|| (%s n=%d)" % (dt.__name__, n))
            # the strict upper triangle is never read
            P = A.copy()
            iu = np.triu_indices(n, 1)
            P[:, iu[0], iu[1]] = dt(7.5)
            d2, e2, Q2 = oracle.sytrd(P, libpath=libpath)
            _fail(out, np.array_equal(d2, d) and np.array_equal(e2, e) and
                  np.array_equal(Q2, Q), "sytrd read the upper triangle (%s n=%d)"
                  % (dt.__name__, n))
            # a tridiagonal matrix is already reduced: T = A, Q = I exactly
            td, te = W.random_batch(n, 4, dt, salt=52)
            Tm = W.dense_from_bands(td, te)
            d3, e3, Q3 = oracle.sytrd(Tm, libpath=libpath)
            _fail(out, np.array_equal(d3, td) and np.array_equal(e3, te) and
                  np.array_equal(Q3, np.broadcast_to(np.eye(n, dtype=dt), Q3.shape)),
                  "sytrd changed a tridiagonal matrix (%s n=%d)" % (dt.__name__, n))
    return out


def pin_syev(oracle, libpath: Optional[str] = None, quick: bool = False) -> List[str]:
    out: List[str] = []
    for dt in (np.float32, np.float64):
        for n in ((3, 16) if quick else (1, 2, 3, 5, 8, 13, 16, 32)):
            A = W.random_symmetric(n, 16, dt, salt=53)
            lam, Q, info = oracle.syev(A, libpath=libpath)
            tol = V.tol_of(dt, n)
            As = _sym_from_lower(A)
            an = np.abs(As).sum(1).max(1)
            _fail(out, not info.any(), "syev info != 0 (%s n=%d)" % (dt.__name__, n))
            ref = np.linalg.eigvalsh(As)
            _fail(out, np.all(np.abs(lam.astype(np.float64) - ref).max(1) <= tol * an),
                  "syev eigenvalues vs eigvalsh (%s n=%d)" % (dt.__name__, n))
            _fail(out, V.dense_residual(As, lam, Q).max() <= tol,
                  "syev residual (%s n=%d)" % (dt.__name__, n))
            _fail(out, V.orthogonality(Q).max() <= tol, "syev orthogonality (%s n=%d)"
                  % (dt.__name__, n))
            td, te = W.random_batch(n, 6, dt, salt=54)
            l1, Q1, i1 = oracle.syev(W.dense_from_bands(td, te), libpath=libpath)
            l2, Q2, i2, _ = oracle.steqr(td, te, True, libpath=libpath)
            _fail(out, np.array_equal(l1, l2) and np.array_equal(Q1, Q2) and
                  np.array_equal(i1, i2), "syev of a tridiagonal A != steqr (%s n=%d)"
                  % (dt.__name__, n))
            dg = W.random_batch(n, 3, dt, salt=55)[0]
            Dm = np.zeros((3, n, n), dtype=dt)
            Dm[:, np.arange(n), np.arange(n)] = dg
            l3, Q3, _ = oracle.syev(Dm, libpath=libpath)
            _fail(out, np.array_equal(l3, np.sort(dg, axis=1)) and
                  np.all(np.abs(Q3).sum(1) == 1) and np.all(np.abs(Q3).sum(2) == 1) and
                  np.all(np.isin(Q3, (0, 1))), "syev of a diagonal A (%s n=%d)"
                  % (dt.__name__, n))
    return out


def pin_stebz(oracle, libpath: Optional[str] = None) -> List[str]:
    out: List[str] = []
    g = np.random.default_rng(71)
    for dt in (np.float32, np.float64):
        # Sturm counts at random points at least 1e-3 ||T|| from every eigenvalue
        for n in (1, 2, 5, 16, 40):
            d, e = W.random_batch(n, 6, dt, salt=72)
            ref = np.linalg.eigvalsh(W.dense_from_bands(d.astype(np.float64), e.astype(np.float64)))
            for b in range(6):
                tn = V.tnorm1(d[b:b + 1], e[b:b + 1])[0]
                pivmin = float(np.finfo(dt).tiny) * max(1.0, float((e[b].astype(np.float64) ** 2).max(initial=0)))
                for x in g.uniform(-1.2 * tn, 1.2 * tn, 12):
                    if np.abs(ref[b] - x).min() < 1e-3 * tn:
                        continue
                    c = oracle.sturm_count(d[b], e[b], dt(x), pivmin, libpath=libpath)
                    _fail(out, c == int((ref[b] < dt(x)).sum()), "Sturm count %s n=%d at %g: %d"
                          % (dt.__name__, n, x, c))
        for n in (1, 2, 3, 8, 13, 16, 32, 64):
            d, e = W.random_batch(n, 24, dt, salt=73)
            lam, info = oracle.stebz(d, e, libpath=libpath)
            tol = V.tol_of(dt, n)
            _fail(out, not info.any(), "stebz info (%s n=%d)" % (dt.__name__, n))
            ref = np.linalg.eigvalsh(W.dense_from_bands(d.astype(np.float64), e.astype(np.float64)))
            _fail(out, V.sorted_err(lam, ref, d, e).max() <= tol,
                  "stebz vs eigvalsh (%s n=%d)" % (dt.__name__, n))
            _fail(out, np.all(np.diff(lam, axis=1) >= 0), "stebz not ascending")
            lq, _, _, _ = oracle.steqr(d, e, False, libpath=libpath)
            _fail(out, V.sorted_err(lam, lq.astype(np.float64), d, e).max() <= tol,
                  "stebz vs the QR solve (%s n=%d)" % (dt.__name__, n))
            for j in (-40, 7, 60):
                ls, _ = oracle.stebz(d * dt(2.0 ** j), e * dt(2.0 ** j), libpath=libpath)
                _fail(out, np.array_equal(ls, lam * dt(2.0 ** j)),
                      "stebz power-of-two scaling (%s n=%d, 2^%d)" % (dt.__name__, n, j))
        for n in (4, 16, 33, 64):
            d, e, ref = clement(n)
            lam, info = oracle.stebz(d.astype(dt), e.astype(dt), libpath=libpath)
            err = np.abs(lam[0].astype(np.float64) - ref).max() / V.tnorm1(d, e)[0]
            _fail(out, info[0] == 0 and err <= V.tol_of(dt, n), "stebz Clement n=%d %s: %g"
                  % (n, dt.__name__, err))
            a, b = 0.5, -1.25
            k = np.arange(1, n + 1)
            tz = np.sort(a + 2 * b * np.cos(k * np.pi / (n + 1)))
            lam, _ = oracle.stebz(np.full((1, n), a, dtype=dt), np.full((1, n - 1), b, dtype=dt),
                                  libpath=libpath)
            _fail(out, np.abs(lam[0] - tz).max() <= V.tol_of(dt, n) * (abs(a) + 2 * abs(b)),
                  "stebz Toeplitz n=%d %s" % (n, dt.__name__))
        dg = W.random_batch(9, 4, dt, salt=74)[0]
        lam, _ = oracle.stebz(dg, np.zeros((4, 8), dtype=dt), libpath=libpath)
        _fail(out, np.all(np.abs(lam - np.sort(dg, 1)) <= V.tol_of(dt, 9) *
                          np.abs(dg).max(1, keepdims=True)), "stebz diagonal T (%s)" % dt.__name__)
        lam, info = oracle.stebz(np.zeros((2, 7), dtype=dt), np.zeros((2, 6), dtype=dt),
                                 libpath=libpath)
        _fail(out, np.all(lam == 0) and not info.any(), "stebz T = 0")
        d, e = W.random_batch(7, 2, dt, salt=75)
        d[0, 3] = np.nan
        e[1, 2] = np.nan
        lam, info = oracle.stebz(d, e, libpath=libpath)
        _fail(out, np.all(np.isnan(lam)) and np.all(info == 7), "stebz NaN")
    return out


ALL_PINS = (pin_lartg, pin_shift, pin_sym2x2, pin_sweep, pin_solve, pin_direction,
            pin_block2, pin_back_transform,
            pin_larfg, pin_sytrd, pin_syev, pin_stebz)


def run_all(oracle, libpath: Optional[str] = None, quick: bool = True) -> List[str]:
    """Every pin; the sweep and whole-solve pins for both update schemes."""
    fails: List[str] = []
    for p in ALL_PINS:
        multi = p in (pin_sweep, pin_solve, pin_direction, pin_block2, pin_back_transform)
        for scheme in ((0, 1) if multi else (0,)):
            try:
                if p in (pin_solve, pin_direction, pin_block2, pin_back_transform):
                    for shift in (0, 1):
                        fails += [f + " [scheme %d, shift %d]" % (scheme, shift)
                                  for f in p(oracle, libpath, quick=quick, scheme=scheme,
                                             shift=shift)]
                elif p is pin_sweep:
                    fails += [f + " [scheme %d]" % scheme for f in p(oracle, libpath, scheme=scheme)]
                else:
                    fails += p(oracle, libpath)
            except Exception as exc:  # a crash of the oracle is a failed pin too
                fails.append("%s raised %r" % (p.__name__, exc))
    return fails
