"""ctypes binding of libsteqr.so (include/steqr.h).

Argument marshalling only: every step of the solve runs in the HIP
kernels. PyTorch supplies device memory and the stream. If the library is
missing this module raises at import; there is no fallback path.
"""
from __future__ import annotations

import ctypes as ct
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsteqr.so")

STEQR_N, STEQR_V = 0, 1
STEQR_F32, STEQR_F64 = 0, 1
STEQR_EXP, STEQR_PG = 0, 1
STEQR_SHIFT_LAPACK, STEQR_SHIFT_CLOSED = 0, 1
STEQR_METHOD_QR, STEQR_METHOD_BISECT = 0, 1
STEQR_MAX_N = 512
SYEV_MAX_N = 32
SYEV_MAX_N_F64_V = 32


class steqr_params(ct.Structure):
    _fields_ = [("max_sweeps_per_n", ct.c_int),
                ("no_sort", ct.c_int),
                ("lanes_per_problem", ct.c_int),
                ("waves_per_block", ct.c_int),
                ("band_storage", ct.c_int),
                ("update_scheme", ct.c_int),
                ("shift", ct.c_int),
                ("back_transform", ct.c_int),
                ("method", ct.c_int)]


class SteqrError(RuntimeError):
    def __init__(self, rc: int, where: str):
        super().__init__("%s returned %d" % (where, rc))
        self.rc = rc


if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsteqr.so is not built (%s); run `python -c \"import __graft_entry__ as g; "
        "g.build()\"` or `python -m symmetric_tridiagonal_eigensolver_amd.build`" % LIB_PATH)

_lib = ct.CDLL(LIB_PATH)
_vp, _i = ct.c_void_p, ct.c_int
_lib.steqr_batched.restype = _i
_lib.steqr_batched.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
_lib.steqr_batched_ex.restype = _i
_lib.steqr_batched_ex.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp,
                                  ct.POINTER(steqr_params)]
_lib.steqr_query.restype = _i
_lib.steqr_query.argtypes = [_i, _i, _i, _i, ct.POINTER(steqr_params)] + [ct.POINTER(_i)] * 6
_lib.steqr_version.restype = ct.c_char_p
_lib.steqr_version.argtypes = []
_lib.syev_batched.restype = _i
_lib.syev_batched.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp]
_lib.syev_batched_ex.restype = _i
_lib.syev_batched_ex.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp,
                                 ct.POINTER(steqr_params)]
_lib.syev_query.restype = _i
_lib.syev_query.argtypes = [_i, _i, _i, _i, ct.POINTER(steqr_params)] + [ct.POINTER(_i)] * 6

EXPORTS = ("steqr_batched", "steqr_batched_ex", "steqr_query", "steqr_version",
           "syev_batched", "syev_batched_ex", "syev_query")


def lib() -> ct.CDLL:
    return _lib


def version() -> str:
    return _lib.steqr_version().decode()


def make_params(max_sweeps_per_n: int = 0, sort: bool = True, lanes_per_problem: int = 0,
                waves_per_block: int = 0, band_storage: int = 0,
                update_scheme: int = 0, shift: int = 0,
                back_transform: bool = False, method: int = 0) -> steqr_params:
    return steqr_params(int(max_sweeps_per_n), 0 if sort else 1, int(lanes_per_problem),
                        int(waves_per_block), int(band_storage), int(update_scheme),
                        int(shift), int(bool(back_transform)), int(method))


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def steqr_batched(d, e, lam, Q, n: int, batch: int, jobz: int, dtype: int, stream=None) -> int:
    """Thin call of the C entry point; returns its status code."""
    return _lib.steqr_batched(_ptr(d), _ptr(e), _ptr(lam), _ptr(Q), int(n), int(batch),
                              int(jobz), int(dtype), _stream_handle(stream))


def steqr_batched_ex(d, e, lam, Q, n: int, batch: int, jobz: int, dtype: int, stream=None,
                     info=None, params: Optional[steqr_params] = None) -> int:
    return _lib.steqr_batched_ex(_ptr(d), _ptr(e), _ptr(lam), _ptr(Q), int(n), int(batch),
                                 int(jobz), int(dtype), _stream_handle(stream), _ptr(info),
                                 ct.byref(params) if params is not None else None)


def steqr_query(n: int, batch: int, jobz: int, dtype: int,
                params: Optional[steqr_params] = None) -> dict:
    outs = [ct.c_int(0) for _ in range(6)]
    rc = _lib.steqr_query(int(n), int(batch), int(jobz), int(dtype),
                          ct.byref(params) if params is not None else None,
                          *[ct.byref(o) for o in outs])
    if rc != 0:
        raise SteqrError(rc, "steqr_query")
    keys = ("padded_n", "lanes_per_problem", "rows_per_lane", "waves_per_block", "workgroups",
            "band_storage")
    return dict(zip(keys, (o.value for o in outs)))


def dtype_code(tdtype) -> int:
    import torch
    if tdtype == torch.float32:
        return STEQR_F32
    if tdtype == torch.float64:
        return STEQR_F64
    raise TypeError("steqr supports float32 and float64, got %s" % tdtype)


def solve(d, e, jobz: bool = True, *, info: bool = False, sort: bool = True,
          max_sweeps_per_n: int = 0, lanes_per_problem: int = 0, waves_per_block: int = 0,
          band_storage: int = 0, update_scheme: int = 0, shift: int = 0, stream=None,
          out: Optional[Tuple] = None, Z=None, method: int = 0):
    """Solve a batch held in device tensors d (batch, n), e (batch, n-1).

    Z: optional (batch, n, n) device basis for back-transformation; it is
    overwritten in place with Z times the rotations and returned as Q.
    Returns (lam, Q or None[, info]) as device tensors; the work is enqueued
    on `stream` (default: torch's current stream) and not synchronised.
    """
    import torch
    if d.dim() != 2 or e.dim() != 2:
        raise ValueError("d must be (batch, n) and e (batch, n-1)")
    batch, n = d.shape
    if e.shape != (batch, max(n - 1, 0)) or e.dtype != d.dtype or e.device != d.device:
        raise ValueError("e must be (batch, n-1) with d's dtype and device")
    if not (d.is_cuda and d.is_contiguous() and e.is_contiguous()):
        raise ValueError("d and e must be contiguous device tensors")
    if out is not None:
        lam, Q, inf = out
    else:
        lam = torch.empty_like(d)
        Q = torch.empty((batch, n, n), dtype=d.dtype, device=d.device) if jobz else None
        inf = torch.empty((batch,), dtype=torch.int32, device=d.device) if info else None
    if Z is not None:
        if not jobz:
            raise ValueError("back-transformation needs jobz")
        if Z.shape != (batch, n, n) or Z.dtype != d.dtype or Z.device != d.device \
                or not Z.is_contiguous():
            raise ValueError("Z must be a contiguous (batch, n, n) device tensor of d's dtype")
        Q = Z
    prm = make_params(max_sweeps_per_n, sort, lanes_per_problem, waves_per_block, band_storage,
                      update_scheme, shift, Z is not None, method)
    rc = steqr_batched_ex(d, e, lam, Q, n, batch, STEQR_V if jobz else STEQR_N,
                          dtype_code(d.dtype), stream, inf, prm)
    if rc != 0:
        raise SteqrError(rc, "steqr_batched_ex")
    return (lam, Q, inf) if info else (lam, Q)


def syev_batched(A, lam, Q, n: int, batch: int, jobz: int, dtype: int, stream=None) -> int:
    """Thin call of the C entry point; returns its status code."""
    return _lib.syev_batched(_ptr(A), _ptr(lam), _ptr(Q), int(n), int(batch), int(jobz),
                             int(dtype), _stream_handle(stream))


def syev_batched_ex(A, lam, Q, n: int, batch: int, jobz: int, dtype: int, stream=None,
                    info=None, params: Optional[steqr_params] = None) -> int:
    return _lib.syev_batched_ex(_ptr(A), _ptr(lam), _ptr(Q), int(n), int(batch), int(jobz),
                                int(dtype), _stream_handle(stream), _ptr(info),
                                ct.byref(params) if params is not None else None)


def syev_query(n: int, batch: int, jobz: int, dtype: int,
               params: Optional[steqr_params] = None) -> dict:
    outs = [ct.c_int(0) for _ in range(6)]
    rc = _lib.syev_query(int(n), int(batch), int(jobz), int(dtype),
                         ct.byref(params) if params is not None else None,
                         *[ct.byref(o) for o in outs])
    if rc != 0:
        raise SteqrError(rc, "syev_query")
    keys = ("padded_n", "lanes_per_problem", "rows_per_lane", "waves_per_block", "workgroups",
            "band_storage")
    return dict(zip(keys, (o.value for o in outs)))


def syev(A, jobz: bool = True, *, info: bool = False, sort: bool = True,
         max_sweeps_per_n: int = 0, lanes_per_problem: int = 0, waves_per_block: int = 0,
         shift: int = 0, band_storage: int = 0, stream=None):
    """Eigen-decomposition of a batch of dense symmetric matrices A (batch, n, n)
    held in a device tensor (lower triangle read). Returns (lam, Q or None[, info])
    as device tensors; the work is enqueued on `stream` and not synchronised."""
    import torch
    if A.dim() != 3 or A.shape[1] != A.shape[2]:
        raise ValueError("A must be (batch, n, n)")
    if not (A.is_cuda and A.is_contiguous()):
        raise ValueError("A must be a contiguous device tensor")
    batch, n = A.shape[0], A.shape[1]
    lam = torch.empty((batch, n), dtype=A.dtype, device=A.device)
    Q = torch.empty_like(A) if jobz else None
    inf = torch.empty((batch,), dtype=torch.int32, device=A.device) if info else None
    prm = make_params(max_sweeps_per_n, sort, lanes_per_problem, waves_per_block, band_storage, 0,
                      shift)
    rc = syev_batched_ex(A, lam, Q, n, batch, STEQR_V if jobz else STEQR_N, dtype_code(A.dtype),
                         stream, inf, prm)
    if rc != 0:
        raise SteqrError(rc, "syev_batched_ex")
    return (lam, Q, inf) if info else (lam, Q)
