"""GPU-vs-oracle parity checks (test infrastructure).

run_gpu() calls the HIP library through its C ABI (via the Python
binding); check() compares its outputs with the CPU oracle's on the same
inputs, item by item:
  * status: the same items fail (info > 0) on both sides, with equal info;
  * converged items: sorted eigenvalues within 16 n eps ||T||_1, and for
    jobz=V residual ||TQ - Q Lambda||_1/||T||_1 and ||Q^T Q - I||_1 within
    16 n eps (eps = 2^-23 / 2^-52);
  * zero matrices: eigenvalues exactly 0 and Q exactly I;
  * failed items: NaN at the same unsorted positions;
  * converged items with a NaN eigenvalue (orders 1 and 2): NaN on both
    sides.
Eigenvectors are compared through residual and orthogonality only: their
signs (and the basis of a repeated eigenvalue) are not unique.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

import validate as V


def run_gpu(d: np.ndarray, e: np.ndarray, jobz: bool, *, sort: bool = True,
            max_sweeps_per_n: int = 0, lanes: int = 0, waves: int = 0, band: int = 0,
            scheme: int = 0, shift: int = 0, Z: Optional[np.ndarray] = None):
    """Z: optional basis for back-transformation (copied to the device and
    overwritten there; the numpy array is untouched)."""
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    dev = torch.device("cuda:0")
    td = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    te = torch.from_numpy(np.ascontiguousarray(e)).to(dev)
    tz = None if Z is None else torch.from_numpy(np.ascontiguousarray(Z)).to(dev)
    lam, Q, info = st.solve(td, te, jobz, info=True, sort=sort,
                            max_sweeps_per_n=max_sweeps_per_n, lanes_per_problem=lanes,
                            waves_per_block=waves, band_storage=band, update_scheme=scheme,
                            shift=shift, Z=tz)
    torch.cuda.synchronize()
    return (lam.cpu().numpy(), None if Q is None else Q.cpu().numpy(), info.cpu().numpy())


def check_basis(d, e, Z, gpu, ora, tol_factor: float = 16.0) -> List[str]:
    """Back-transformation with an orthogonal basis Z: status and
    eigenvalues as in check(); the columns of the GPU's Q are orthonormal
    eigenvectors of the dense A = Z T Z^T (residual and orthogonality within
    16 n eps); items with T = 0 return Z exactly."""
    out = check(d, e, gpu, ora, False, tol_factor)
    lg, Qg, ig = gpu
    n = d.shape[1]
    tol = V.tol_of(d.dtype, n, tol_factor)
    ok = (ig == 0) & (ora[2] == 0) & ~np.isnan(lg).any(axis=1)
    if ok.any():
        Z64 = Z[ok].astype(np.float64)
        import workloads as W
        A = np.matmul(np.matmul(Z64, W.dense_from_bands(d[ok].astype(np.float64),
                                                        e[ok].astype(np.float64))),
                      np.swapaxes(Z64, 1, 2))
        res = V.dense_residual(A, lg[ok], Qg[ok])
        if not (res.max() <= tol):
            out.append("dense residual %.3g > tol %.3g" % (res.max(), tol))
        orth = V.orthogonality(Qg[ok])
        if not (orth.max() <= tol):
            out.append("orthogonality %.3g > tol %.3g" % (orth.max(), tol))
        zero = ok & (V.tnorm1(d, e) == 0)
        if zero.any() and not np.array_equal(Qg[zero], Z[zero]):
            out.append("zero matrix: Q is not the basis")
    return out


def check(d, e, gpu, ora, jobz: bool, tol_factor: float = 16.0,
          items: Optional[np.ndarray] = None) -> List[str]:
    """Compare gpu = (lam, Q, info) with ora = (lam, Q, info) on items
    (indices into d/e; default all). gpu arrays may hold more items than
    ora: gpu[items[k]] pairs with ora[k]."""
    out: List[str] = []
    lg, Qg, ig = gpu
    lo, Qo, io = ora[:3]
    if items is None:
        items = np.arange(d.shape[0])
    d, e = d[items], e[items]
    lg, ig = lg[items], ig[items]
    if Qg is not None:
        Qg = Qg[items]
    n = d.shape[1]
    tol = V.tol_of(d.dtype, n, tol_factor)
    fail_g, fail_o = ig > 0, io > 0
    if not np.array_equal(fail_g, fail_o):
        bad = np.nonzero(fail_g != fail_o)[0][:8]
        out.append("status differs at items %s (gpu info %s, oracle %s)"
                   % (items[bad].tolist(), ig[bad].tolist(), io[bad].tolist()))
    both_fail = fail_g & fail_o
    if both_fail.any():
        if not np.array_equal(ig[both_fail], io[both_fail]):
            out.append("info counts differ on failed items")
        if not np.array_equal(np.isnan(lg[both_fail]), np.isnan(lo[both_fail])):
            out.append("NaN positions differ on failed items")
    # converged items that carry a NaN (orders 1 and 2 reach no iteration
    # that could fail): NaN on both sides, nothing else to compare
    nan_g = ~fail_g & np.isnan(lg).any(axis=1)
    nan_o = ~fail_o & np.isnan(lo).any(axis=1)
    if not np.array_equal(nan_g, nan_o):
        out.append("NaN eigenvalues differ on converged items %s"
                   % items[nan_g != nan_o][:8].tolist())
    ok = ~fail_g & ~fail_o & ~nan_g & ~nan_o
    if ok.any():
        err = V.sorted_err(lg[ok], lo[ok], d[ok], e[ok])
        if not (err.max() <= tol):
            k = int(np.argmax(err))
            out.append("eigenvalues: max err %.3g > tol %.3g (item %d)"
                       % (err.max(), tol, int(items[ok][k])))
        if not np.all(np.diff(lg[ok], axis=1) >= 0):
            out.append("gpu eigenvalues not ascending")
        if jobz:
            res = V.band_residual(d[ok], e[ok], lg[ok], Qg[ok])
            if not (res.max() <= tol):
                out.append("residual %.3g > tol %.3g" % (res.max(), tol))
            orth = V.orthogonality(Qg[ok])
            if not (orth.max() <= tol):
                out.append("orthogonality %.3g > tol %.3g" % (orth.max(), tol))
        zero = ok & (V.tnorm1(d, e) == 0)
        if zero.any():
            if not np.all(lg[zero] == 0):
                out.append("zero matrix: eigenvalues not exactly 0")
            if jobz and not np.array_equal(Qg[zero], np.broadcast_to(np.eye(n), Qg[zero].shape)):
                out.append("zero matrix: Q not exactly I")
    return out


def sym_from_lower(A) -> np.ndarray:
    """The symmetric matrix a dense solver sees: lower triangle of A,
    mirrored (float64)."""
    L = np.tril(np.asarray(A, dtype=np.float64))
    return L + np.swapaxes(np.tril(L, -1), 1, 2)


def run_gpu_syev(A: np.ndarray, jobz: bool, *, sort: bool = True, max_sweeps_per_n: int = 0,
                 lanes: int = 0, waves: int = 0, shift: int = 0, band: int = 0):
    import torch
    import symmetric_tridiagonal_eigensolver_amd as st
    tA = torch.from_numpy(np.ascontiguousarray(A)).to(torch.device("cuda:0"))
    lam, Q, info = st.syev(tA, jobz, info=True, sort=sort, max_sweeps_per_n=max_sweeps_per_n,
                           lanes_per_problem=lanes, waves_per_block=waves, shift=shift,
                           band_storage=band)
    torch.cuda.synchronize()
    return (lam.cpu().numpy(), None if Q is None else Q.cpu().numpy(), info.cpu().numpy())


def check_dense(A, gpu, ora, jobz: bool, tol_factor: float = 16.0,
                sort: bool = True) -> List[str]:
    """Dense solver parity: the same items fail with equal info; converged
    items have sorted eigenvalues within 16 n eps ||A||_1 of the oracle's,
    and with eigenvectors the dense residual ||AQ - Q Lambda||_1/||A||_1
    and ||Q^T Q - I||_1 within 16 n eps; zero matrices give lambda = 0 and
    Q = I exactly; NaN items NaN on both sides."""
    out: List[str] = []
    lg, Qg, ig = gpu
    lo, Qo, io = ora[:3]
    n = A.shape[1]
    tol = V.tol_of(A.dtype, n, tol_factor)
    As = sym_from_lower(A)
    an = np.abs(As).sum(axis=1).max(axis=1)
    if not np.array_equal(ig > 0, io > 0):
        bad = np.nonzero((ig > 0) != (io > 0))[0][:8]
        out.append("status differs at items %s" % bad.tolist())
    nan_g = np.isnan(lg).any(axis=1)
    nan_o = np.isnan(lo).any(axis=1)
    if not np.array_equal(nan_g, nan_o):
        out.append("NaN items differ: %s" % np.nonzero(nan_g != nan_o)[0][:8].tolist())
    ok = (ig == 0) & (io == 0) & ~nan_g & ~nan_o
    if ok.any():
        err = np.abs(np.sort(lg[ok].astype(np.float64), 1) - np.sort(lo[ok].astype(np.float64), 1))
        rel = err.max(axis=1) / np.where(an[ok] > 0, an[ok], 1.0)
        if not (rel.max() <= tol):
            out.append("eigenvalues: max err %.3g > tol %.3g (item %d)"
                       % (rel.max(), tol, int(np.nonzero(ok)[0][np.argmax(rel)])))
        if sort and not np.all(np.diff(lg[ok], axis=1) >= 0):
            out.append("gpu eigenvalues not ascending")
        if jobz:
            res = V.dense_residual(As[ok], lg[ok], Qg[ok])
            if not (res.max() <= tol):
                out.append("dense residual %.3g > tol %.3g" % (res.max(), tol))
            orth = V.orthogonality(Qg[ok])
            if not (orth.max() <= tol):
                out.append("orthogonality %.3g > tol %.3g" % (orth.max(), tol))
        zero = ok & (an == 0)
        if zero.any():
            if not np.all(lg[zero] == 0):
                out.append("zero matrix: eigenvalues not exactly 0")
            if jobz and not np.array_equal(Qg[zero], np.broadcast_to(np.eye(n), Qg[zero].shape)):
                out.append("zero matrix: Q not exactly I")
    return out
