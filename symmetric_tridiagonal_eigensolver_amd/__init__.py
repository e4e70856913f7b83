"""MI355X-native batched symmetric tridiagonal eigensolver (small-n steqr),
and the fused small-n dense symmetric eigensolver built on it (syev).

The solver is the HIP library libsteqr.so (C ABI in include/steqr.h);
this package is its Python binding. Importing it requires the library to
be built (``python -m symmetric_tridiagonal_eigensolver_amd.build``).
"""
from ._binding import (STEQR_METHOD_BISECT, STEQR_METHOD_QR, STEQR_EXP, STEQR_F32, STEQR_F64, STEQR_MAX_N, STEQR_N, STEQR_PG,
                       STEQR_SHIFT_CLOSED, STEQR_SHIFT_LAPACK, STEQR_V, EXPORTS,
                       LIB_PATH, SteqrError, dtype_code, lib, make_params, solve,
                       steqr_batched, steqr_batched_ex, steqr_params, steqr_query, version,
                       SYEV_MAX_N, SYEV_MAX_N_F64_V, syev, syev_batched, syev_batched_ex,
                       syev_query)

__all__ = ["STEQR_METHOD_QR", "STEQR_METHOD_BISECT", "STEQR_EXP", "STEQR_PG", "STEQR_SHIFT_LAPACK", "STEQR_SHIFT_CLOSED", "STEQR_F32", "STEQR_F64", "STEQR_MAX_N", "STEQR_N", "STEQR_V", "EXPORTS",
           "LIB_PATH", "SteqrError", "dtype_code", "lib", "make_params", "solve",
           "steqr_batched", "steqr_batched_ex", "steqr_params", "steqr_query", "version",
           "SYEV_MAX_N", "SYEV_MAX_N_F64_V", "syev", "syev_batched", "syev_batched_ex",
           "syev_query"]
