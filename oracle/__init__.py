"""CPU oracle for the batched symmetric tridiagonal eigensolver.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and
the benchmark's CPU-baseline leg may import this package. The GPU library
and its Python binding never import, link or call it, and it shares no code
with them.

The solver itself is plain C (``steqr_oracle_impl.h``), an implicit shifted
QR/QL iteration written step by step from the BatchLAS steqr algorithm page
(deflation, scaling, shift, Givens bulge chase, split bookkeeping,
eigenvector accumulation, sort), and the dense front end of the fused
small-n syev (``syev_oracle_impl.h``: Householder reduction to tridiagonal
form, then that solve with back-transformation) and the values-only
bisection (``stebz_oracle_impl.h``: Sturm counts, one eigenvalue index at
a time). It runs in the item's precision with IEEE
semantics and no FMA contraction. This module builds it with gcc, loads it
with ctypes and splits batches across threads (ctypes releases the GIL while
the C code runs).
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes as _ct
import os as _os
import subprocess as _sp
from typing import Optional, Tuple

import numpy as _np

HERE = _os.path.dirname(_os.path.abspath(__file__))
SOURCE = _os.path.join(HERE, "steqr_oracle.c")
IMPL = _os.path.join(HERE, "steqr_oracle_impl.h")
IMPL_SYEV = _os.path.join(HERE, "syev_oracle_impl.h")
IMPL_STEBZ = _os.path.join(HERE, "stebz_oracle_impl.h")
LIBNAME = "liboracle_steqr.so"
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_libs = {}


def build(out_dir: str = HERE, source_dir: str = HERE, extra_flags=()) -> str:
    """Compile the oracle library with gcc and return its path."""
    out = _os.path.join(out_dir, LIBNAME)
    tmp = out + ".tmp%d" % _os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp,
           _os.path.join(source_dir, "steqr_oracle.c"), "-lm"]
    _sp.run(cmd, check=True)
    _os.replace(tmp, out)
    return out


def _stale(path: str) -> bool:
    if not _os.path.exists(path):
        return True
    t = _os.path.getmtime(path)
    return any(_os.path.getmtime(s) > t for s in (SOURCE, IMPL, IMPL_SYEV, IMPL_STEBZ))


def lib(path: Optional[str] = None) -> _ct.CDLL:
    """Load (building first if absent or older than its sources)."""
    if path is None:
        path = _os.path.join(HERE, LIBNAME)
        if _stale(path):
            build()
    if path not in _libs:
        L = _ct.CDLL(path)
        for sfx, ct in (("f32", _ct.c_float), ("f64", _ct.c_double)):
            P = _ct.POINTER(ct)
            f = getattr(L, "oracle_steqr_batched_" + sfx)
            f.restype = _ct.c_int
            f.argtypes = [_ct.c_void_p] * 6 + [_ct.c_int, _ct.c_long, _ct.c_int, _ct.c_int,
                                               _ct.c_int, _ct.c_int, _ct.c_int]
            f = getattr(L, "oracle_lartg_" + sfx)
            f.restype = None
            f.argtypes = [ct, ct, P, P, P]
            for name in ("oracle_shift_", "oracle_shift_closed_"):
                f = getattr(L, name + sfx)
                f.restype = ct
                f.argtypes = [ct, ct, ct]
            f = getattr(L, "oracle_sym2x2_" + sfx)
            f.restype = None
            f.argtypes = [ct, ct, ct, P, P, P, P]
            for name in ("oracle_sweep_", "oracle_sweep_pg_"):
                f = getattr(L, name + sfx)
                f.restype = _ct.c_long
                f.argtypes = [_ct.c_void_p, _ct.c_void_p, _ct.c_void_p, _ct.c_int,
                              _ct.c_int, _ct.c_int, ct]
            f = getattr(L, "oracle_constants_" + sfx)
            f.restype = None
            f.argtypes = [_ct.c_void_p]
            f = getattr(L, "oracle_larfg_" + sfx)
            f.restype = None
            f.argtypes = [_ct.c_int, ct, _ct.c_void_p, P, P]
            f = getattr(L, "oracle_sytrd_batched_" + sfx)
            f.restype = _ct.c_int
            f.argtypes = [_ct.c_void_p] * 4 + [_ct.c_int, _ct.c_long]
            f = getattr(L, "oracle_sturm_count_" + sfx)
            f.restype = _ct.c_int
            f.argtypes = [_ct.c_int, _ct.c_void_p, _ct.c_void_p, ct, ct]
            f = getattr(L, "oracle_stebz_batched_" + sfx)
            f.restype = _ct.c_int
            f.argtypes = [_ct.c_void_p] * 5 + [_ct.c_int, _ct.c_long]
            f = getattr(L, "oracle_syev_batched_" + sfx)
            f.restype = _ct.c_int
            f.argtypes = [_ct.c_void_p] * 4 + [_ct.c_int, _ct.c_long, _ct.c_int, _ct.c_int,
                                               _ct.c_int, _ct.c_int]
        _libs[path] = L
    return _libs[path]


def _sfx(dtype) -> str:
    dt = _np.dtype(dtype)
    if dt == _np.float32:
        return "f32"
    if dt == _np.float64:
        return "f64"
    raise TypeError("oracle supports float32 and float64, got %s" % dt)


def _ptr(a: Optional[_np.ndarray]):
    return None if a is None else a.ctypes.data


def steqr(d: _np.ndarray, e: _np.ndarray, jobz: bool = True,
          max_sweeps_per_n: int = 30, sort: bool = True, threads: int = 1,
          libpath: Optional[str] = None, scheme: int = 0, shift: int = 0,
          Z: Optional[_np.ndarray] = None
          ) -> Tuple[_np.ndarray, Optional[_np.ndarray], _np.ndarray, _np.ndarray]:
    """Solve a batch. d: (batch, n), e: (batch, n-1), same float dtype.
    scheme: 0 = EXP sweeps (local similarities), 1 = PG (Parlett-Gray) sweeps.
    shift: 0 = LAPACK-form shift, 1 = closed-form lambda+- shift.
    Z: None (Q starts as the identity) or a (batch, n, n) row-major basis of
    the same dtype (back-transformation: Q = Z times the rotations; needs
    jobz). Z itself is not modified.

    Returns (lam (batch, n), Q (batch, n, n) or None, info (batch,) int32,
    stats (batch, 3) int64 = [implicit sweeps, sweep rotations, 2x2 solves]).
    """
    d = _np.ascontiguousarray(d)
    e = _np.ascontiguousarray(e)
    if d.ndim != 2 or e.ndim != 2 or e.shape[0] != d.shape[0] or \
            e.shape[1] != max(d.shape[1] - 1, 0) or e.dtype != d.dtype:
        raise ValueError("bad band shapes %s %s" % (d.shape, e.shape))
    batch, n = d.shape
    sfx = _sfx(d.dtype)
    lam = _np.empty_like(d)
    Q = _np.empty((batch, n, n), dtype=d.dtype) if jobz else None
    if Z is not None:
        if not jobz:
            raise ValueError("back-transformation needs eigenvectors (jobz)")
        if Z.shape != (batch, n, n) or Z.dtype != d.dtype:
            raise ValueError("bad basis shape %s / dtype %s" % (Z.shape, Z.dtype))
        Q[...] = Z
    info = _np.zeros(batch, dtype=_np.int32)
    stats = _np.zeros((batch, 3), dtype=_np.int64)
    if batch == 0 or n == 0:
        return lam, Q, info, stats
    fn = getattr(lib(libpath), "oracle_steqr_batched_" + sfx)
    it = d.itemsize

    def run(lo: int, hi: int) -> int:
        cnt = hi - lo
        return fn(d.ctypes.data + lo * n * it,
                  e.ctypes.data + lo * max(n - 1, 0) * it,
                  lam.ctypes.data + lo * n * it,
                  None if Q is None else Q.ctypes.data + lo * n * n * it,
                  info.ctypes.data + lo * 4,
                  stats.ctypes.data + lo * 3 * 8,
                  n, cnt, int(max_sweeps_per_n), int(bool(sort)), int(scheme), int(shift),
                  int(Z is not None))

    threads = max(1, min(int(threads), batch))
    if threads == 1:
        rc = run(0, batch)
        if rc != 0:
            raise ValueError("oracle rejected n=%d" % n)
    else:
        cuts = [batch * k // threads for k in range(threads + 1)]
        with _cf.ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(lambda k: run(cuts[k], cuts[k + 1]), range(threads)))
        if any(rcs):
            raise ValueError("oracle rejected n=%d" % n)
    return lam, Q, info, stats


def lartg(f: float, g: float, dtype=_np.float64, libpath=None):
    """(c, s, r) with G(c,s)^T (f, g) = (r, 0), G = [[c,-s],[s,c]]."""
    sfx = _sfx(dtype)
    ct = _ct.c_float if sfx == "f32" else _ct.c_double
    c, s, r = ct(), ct(), ct()
    getattr(lib(libpath), "oracle_lartg_" + sfx)(f, g, _ct.byref(c), _ct.byref(s), _ct.byref(r))
    return c.value, s.value, r.value


def shift(d1: float, d2: float, e1: float, dtype=_np.float64, libpath=None,
          closed: bool = False) -> float:
    """Eigenvalue of [[d2, e1], [e1, d1]] nearest d1 (LAPACK-form shift, or
    the closed form lambda+- with closed=True)."""
    name = "oracle_shift_closed_" if closed else "oracle_shift_"
    return getattr(lib(libpath), name + _sfx(dtype))(d1, d2, e1)


def sym2x2(a: float, b: float, c: float, dtype=_np.float64, libpath=None):
    """(rt1, rt2, cs, sn): J^T [[a,b],[b,c]] J = diag(rt1, rt2), J = [[cs,sn],[-sn,cs]]."""
    sfx = _sfx(dtype)
    ct = _ct.c_float if sfx == "f32" else _ct.c_double
    o = [ct() for _ in range(4)]
    getattr(lib(libpath), "oracle_sym2x2_" + sfx)(a, b, c, *[_ct.byref(x) for x in o])
    return tuple(x.value for x in o)


def sweep(d: _np.ndarray, e: _np.ndarray, Q: Optional[_np.ndarray], s: int, m: int,
          mu: float, libpath=None, scheme: int = 0) -> int:
    """One implicit QR sweep on [s, m] in place (d: (n,), e: (n-1,), Q: (n,n)),
    EXP form (scheme 0) or PG form (scheme 1)."""
    n = d.shape[0]
    assert d.flags.c_contiguous and e.flags.c_contiguous
    assert 0 <= s < m < n
    if Q is not None:
        assert Q.flags.c_contiguous and Q.shape == (n, n) and Q.dtype == d.dtype
    name = "oracle_sweep_pg_" if scheme else "oracle_sweep_"
    return getattr(lib(libpath), name + _sfx(d.dtype))(
        d.ctypes.data, e.ctypes.data, _ptr(Q), n, s, m, mu)


def constants(dtype) -> dict:
    """eps, safmin, ssfmax, ssfmin, eps^2 as the oracle computes them."""
    sfx = _sfx(dtype)
    out = _np.zeros(5, dtype=_np.float32 if sfx == "f32" else _np.float64)
    getattr(lib(), "oracle_constants_" + sfx)(out.ctypes.data)
    return dict(zip(("eps", "safmin", "ssfmax", "ssfmin", "eps2"), out.tolist()))


def larfg(alpha: float, x: _np.ndarray, libpath=None):
    """Householder reflector of (alpha, x): returns (beta, tau, v) with v the
    trailing part of the reflector vector (its first entry is 1)."""
    x = _np.array(x, copy=True)
    assert x.ndim == 1 and x.flags.c_contiguous
    ct = _ct.c_float if x.dtype == _np.float32 else _ct.c_double
    beta, tau = ct(), ct()
    getattr(lib(libpath), "oracle_larfg_" + _sfx(x.dtype))(
        x.shape[0], alpha, x.ctypes.data, _ct.byref(beta), _ct.byref(tau))
    return beta.value, tau.value, x


def _dense(A: _np.ndarray):
    A = _np.ascontiguousarray(A)
    if A.ndim != 3 or A.shape[1] != A.shape[2]:
        raise ValueError("A must be (batch, n, n), got %s" % (A.shape,))
    return A, A.shape[0], A.shape[1]


def sytrd(A: _np.ndarray, want_q: bool = True, libpath=None):
    """Householder reduction of each A (lower triangle read) to tridiagonal
    form: returns (d (batch, n), e (batch, n-1), Q (batch, n, n) or None)
    with A = Q T Q^T."""
    A, batch, n = _dense(A)
    d = _np.empty((batch, n), dtype=A.dtype)
    e = _np.empty((batch, max(n - 1, 0)), dtype=A.dtype)
    Q = _np.empty_like(A) if want_q else None
    if batch and n:
        rc = getattr(lib(libpath), "oracle_sytrd_batched_" + _sfx(A.dtype))(
            A.ctypes.data, d.ctypes.data, e.ctypes.data, _ptr(Q), n, batch)
        if rc != 0:
            raise ValueError("oracle rejected n=%d" % n)
    return d, e, Q


def syev(A: _np.ndarray, jobz: bool = True, max_sweeps_per_n: int = 30, sort: bool = True,
         threads: int = 1, libpath: Optional[str] = None, scheme: int = 0, shift: int = 0
         ) -> Tuple[_np.ndarray, Optional[_np.ndarray], _np.ndarray]:
    """Dense symmetric eigensolver: (lam (batch, n) ascending, Q (batch, n, n)
    or None, info (batch,) int32) for each A (lower triangle read)."""
    A, batch, n = _dense(A)
    lam = _np.empty((batch, n), dtype=A.dtype)
    Q = _np.empty_like(A) if jobz else None
    info = _np.zeros(batch, dtype=_np.int32)
    if batch == 0 or n == 0:
        return lam, Q, info
    fn = getattr(lib(libpath), "oracle_syev_batched_" + _sfx(A.dtype))
    it = A.itemsize

    def run(lo: int, hi: int) -> int:
        return fn(A.ctypes.data + lo * n * n * it, lam.ctypes.data + lo * n * it,
                  None if Q is None else Q.ctypes.data + lo * n * n * it,
                  info.ctypes.data + lo * 4, n, hi - lo, int(max_sweeps_per_n),
                  int(bool(sort)), int(scheme), int(shift))

    threads = max(1, min(int(threads), batch))
    cuts = [batch * k // threads for k in range(threads + 1)]
    if threads == 1:
        rcs = [run(0, batch)]
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(lambda k: run(cuts[k], cuts[k + 1]), range(threads)))
    if any(rcs):
        raise ValueError("oracle rejected n=%d" % n)
    return lam, Q, info


def sturm_count(d: _np.ndarray, e: _np.ndarray, x: float, pivmin: float, libpath=None) -> int:
    """Number of eigenvalues of one tridiagonal (d (n,), e (n-1,)) below x."""
    d = _np.ascontiguousarray(d)
    e2 = _np.ascontiguousarray(_np.asarray(e, dtype=d.dtype) ** 2)
    return getattr(lib(libpath), "oracle_sturm_count_" + _sfx(d.dtype))(
        d.shape[0], d.ctypes.data, e2.ctypes.data, x, pivmin)


def stebz(d: _np.ndarray, e: _np.ndarray, threads: int = 1, libpath=None,
          counts: bool = False):
    """Values-only bisection of a batch: (lam (batch, n) ascending, info
    (batch,) = indices that ran out of halvings[, Sturm counts evaluated per
    item (batch,) int64 when counts])."""
    d = _np.ascontiguousarray(d)
    e = _np.ascontiguousarray(e)
    batch, n = d.shape
    if e.shape != (batch, max(n - 1, 0)) or e.dtype != d.dtype:
        raise ValueError("bad band shapes %s %s" % (d.shape, e.shape))
    lam = _np.empty_like(d)
    info = _np.zeros(batch, dtype=_np.int32)
    cnt = _np.zeros(batch, dtype=_np.int64)
    if batch == 0 or n == 0:
        return (lam, info, cnt) if counts else (lam, info)
    fn = getattr(lib(libpath), "oracle_stebz_batched_" + _sfx(d.dtype))
    it = d.itemsize

    def run(lo: int, hi: int) -> int:
        return fn(d.ctypes.data + lo * n * it, e.ctypes.data + lo * max(n - 1, 0) * it,
                  lam.ctypes.data + lo * n * it, info.ctypes.data + lo * 4,
                  cnt.ctypes.data + lo * 8, n, hi - lo)

    threads = max(1, min(int(threads), batch))
    cuts = [batch * k // threads for k in range(threads + 1)]
    if threads == 1:
        rcs = [run(0, batch)]
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(lambda k: run(cuts[k], cuts[k + 1]), range(threads)))
    if any(rcs):
        raise ValueError("oracle rejected n=%d" % n)
    return (lam, info, cnt) if counts else (lam, info)
