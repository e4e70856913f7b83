"""Validators shared by the oracle pins and the GPU parity tests.

Test infrastructure: plain numpy, independent of both the oracle and the
HIP path. Acceptance rule for floating point: sorted
eigenvalues within 16*n*eps*||T||, residual ||TQ - Q Lambda|| / ||T|| and
orthogonality ||Q^T Q - I|| within 16*n*eps, with eps the machine epsilon
of the item's precision (2^-23 for float32, 2^-52 for float64) and ||.||
the 1-norm (max column sum).
"""
from __future__ import annotations

import numpy as np

LD = np.longdouble


def eps_of(dtype) -> float:
    return float(np.finfo(np.dtype(dtype)).eps)


def tol_of(dtype, n: int, factor: float = 16.0) -> float:
    return factor * max(n, 1) * eps_of(dtype)


def tnorm1(d: np.ndarray, e: np.ndarray) -> np.ndarray:
    """1-norm of each tridiagonal: max_i |e_{i-1}| + |d_i| + |e_i| (float64)."""
    d = np.abs(np.asarray(d, dtype=np.float64))
    e = np.abs(np.asarray(e, dtype=np.float64))
    col = d.copy()
    if e.shape[1] > 0:
        col[:, :-1] += e
        col[:, 1:] += e
    return col.max(axis=1)


def band_residual(d, e, lam, Q) -> np.ndarray:
    """||T Q - Q diag(lam)||_1 / ||T||_1 per item, from the bands, in float64.

    (TQ)_ij = e_{i-1} Q_{i-1,j} + d_i Q_ij + e_i Q_{i+1,j}; four terms per
    entry, so the float64 evaluation error is a few eps64 * ||T||, far below
    any tolerance used here. Items with ||T|| = 0 return the absolute value.
    """
    d = np.asarray(d, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    TQ = d[:, :, None] * Q
    if e.shape[1] > 0:
        TQ[:, :-1, :] += e[:, :, None] * Q[:, 1:, :]
        TQ[:, 1:, :] += e[:, :, None] * Q[:, :-1, :]
    R = TQ - Q * lam[:, None, :]
    rn = np.abs(R).sum(axis=1).max(axis=1)
    tn = tnorm1(d, e)
    return np.where(tn > 0, rn / np.where(tn > 0, tn, 1.0), rn)


def dense_residual(A, lam, Q) -> np.ndarray:
    """||A Q - Q diag(lam)||_1 / ||A||_1 per item for dense (batch, n, n) A,
    in float64. Items with ||A|| = 0 return the absolute value."""
    A = np.asarray(A, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    R = np.matmul(A, Q) - Q * lam[:, None, :]
    rn = np.abs(R).sum(axis=1).max(axis=1)
    an = np.abs(A).sum(axis=1).max(axis=1)
    return np.where(an > 0, rn / np.where(an > 0, an, 1.0), rn)


def orthogonality(Q) -> np.ndarray:
    """||Q^T Q - I||_1 per item, in float64."""
    Q = np.asarray(Q, dtype=np.float64)
    n = Q.shape[-1]
    G = np.matmul(np.swapaxes(Q, 1, 2), Q) - np.eye(n)
    return np.abs(G).sum(axis=1).max(axis=1)


def sorted_err(l1, l2, d, e) -> np.ndarray:
    """max_k |sort(l1)_k - sort(l2)_k| / ||T||_1 per item (float64)."""
    a = np.sort(np.asarray(l1, dtype=np.float64), axis=1)
    b = np.sort(np.asarray(l2, dtype=np.float64), axis=1)
    tn = tnorm1(d, e)
    err = np.abs(a - b).max(axis=1) if a.shape[1] else np.zeros(a.shape[0])
    return np.where(tn > 0, err / np.where(tn > 0, tn, 1.0), err)


def sturm_eigvals(d, e, iters: int = 140) -> np.ndarray:
    """All eigenvalues of each tridiagonal by Sturm-count bisection, in
    long double (64-bit mantissa on x86-64).

    count(x) = number of negative pivots of the LDL^T factorisation of
    T - xI: q_1 = d_1 - x, q_i = (d_i - x) - e_{i-1}^2 / q_{i-1}; a zero
    pivot is replaced by -pivmin. The k-th eigenvalue is bisected inside
    the Gershgorin interval until the interval stops shrinking. Vectorised
    over items and over k. Returns long double (batch, n), ascending.
    """
    d = np.asarray(d, dtype=LD)
    e = np.asarray(e, dtype=LD)
    nb, n = d.shape
    ae = np.abs(e)
    rad = np.zeros_like(d)
    if n > 1:
        rad[:, :-1] += ae
        rad[:, 1:] += ae
    lo = (d - rad).min(axis=1)
    hi = (d + rad).max(axis=1)
    span = np.maximum(np.abs(lo), np.abs(hi))
    lo = lo - span * LD(1e-12) - LD(0)
    hi = hi + span * LD(1e-12)
    e2 = e * e
    tiny = np.finfo(LD).tiny
    pivmin = tiny * np.maximum(LD(1), (e2.max(axis=1) if n > 1 else np.ones(nb, dtype=LD)))
    k = np.arange(n)
    L = np.repeat(lo[:, None], n, axis=1)
    H = np.repeat(hi[:, None], n, axis=1)
    for _ in range(iters):
        x = (L + H) / 2
        q = d[:, :1] - x
        q = np.where(q == 0, -pivmin[:, None], q)
        cnt = (q < 0).astype(np.int64)
        for i in range(1, n):
            q = (d[:, i:i + 1] - x) - e2[:, i - 1:i] / q
            q = np.where(np.abs(q) < pivmin[:, None], -pivmin[:, None], q)
            cnt += (q < 0)
        below = cnt > k[None, :]  # at least k+1 eigenvalues < x
        H = np.where(below, x, H)
        L = np.where(below, L, x)
    return (L + H) / 2
