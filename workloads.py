"""Seeded synthetic inputs for the batched symmetric tridiagonal eigensolver.

This module is shared by the tests, the benchmark and the smoke check. It
holds only input construction (random numbers and the edge-item recipes);
none of the solver's arithmetic lives here, so both the HIP path and the
CPU oracle can be fed from it without sharing any of the method.

A matrix is given by its diagonal ``d`` (n entries) and off-diagonal
``e`` (n-1 entries), packed per matrix: ``d`` has shape (batch, n) and
``e`` shape (batch, n-1), as in the BatchLAS steqr algorithm page (the
problem statement and band storage at the top of the page).

Random values are drawn in float64 from
``numpy.random.Generator(PCG64(SeedSequence([1234, cfg, n])))`` and cast to
float32 for float32 runs, so the float32 and float64 items of one
configuration share their base matrices. The pages draw random normal d and
e (BatchLAS "STEQR: the CTA tridiagonal solver" page, setup paragraph) and
use seed 1234 in their accuracy harnesses (BatchLAS "SYCL implementations"
page, accuracy section).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

SEED = 1234

# Edge-item kinds used in the mixed workload (one kind per edge item).
EDGE_SPLIT, EDGE_GRADED, EDGE_ZERO, EDGE_SCALED, EDGE_NAN = range(5)
EDGE_NAMES = ("split", "graded", "zero", "scaled", "nan")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity configuration."""

    cfg: int            # configuration id, part of the seed
    name: str           # short human-readable name
    dtype: str          # "f32" or "f64"
    n: int              # matrix order
    batch: int          # matrices per launch
    jobz: Tuple[str, ...]  # "V" and/or "N"
    lanes: int          # lanes per problem named for the configuration
    edge_mix: bool = False  # 10% edge items (split/graded/zero/scaled/NaN)

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float64


# The five configurations of the pages' CTA benchmarks (sizes, batches and
# lanes per problem), then the work-group orders beyond them. Inputs: d and
# e iid N(0, 1) from the seeded generator below; the C4 configurations mix
# in 10% edge items (one kind per item).
WORKLOADS: Dict[str, Workload] = {
    "c1_f32_n4": Workload(1, "c1_f32_n4", "f32", 4, 4096, ("V",), 4),
    "c2_f32_n8": Workload(2, "c2_f32_n8", "f32", 8, 65536, ("V", "N"), 8),
    "c2_f32_n16": Workload(2, "c2_f32_n16", "f32", 16, 32768, ("V", "N"), 16),
    "c3_f64_n12": Workload(3, "c3_f64_n12", "f64", 12, 32768, ("V",), 16),
    "c3_f64_n16": Workload(3, "c3_f64_n16", "f64", 16, 32768, ("V",), 16),
    "c4_f32_n32": Workload(4, "c4_f32_n32", "f32", 32, 32768, ("V", "N"), 32, True),
    "c4_f64_n32": Workload(4, "c4_f64_n32", "f64", 32, 32768, ("V", "N"), 32, True),
    "c5_f64_n64": Workload(5, "c5_f64_n64", "f64", 64, 16384, ("V",), 64),
    # beyond the sub-group width: the work-group path's orders (65..128)
    "w_f32_n128": Workload(6, "w_f32_n128", "f32", 128, 8192, ("V", "N"), 16),
    "w_f64_n128": Workload(7, "w_f64_n128", "f64", 128, 8192, ("V", "N"), 16),
    "w_f32_n256": Workload(8, "w_f32_n256", "f32", 256, 1024, ("V", "N"), 32),
    "w_f64_n256": Workload(10, "w_f64_n256", "f64", 256, 1024, ("V", "N"), 32),
    "w_f32_n512": Workload(11, "w_f32_n512", "f32", 512, 256, ("V", "N"), 64),
    "w_f64_n512": Workload(12, "w_f64_n512", "f64", 512, 256, ("V", "N"), 64),
}

HEADLINE = "c2_f32_n16"

# Workloads whose small-batch parity tests run the oracle on about a
# thousand items (orders up to 256; at order 512 the oracle takes about a
# second per matrix with eigenvectors, so those workloads are checked on
# samples of the full batch and on seeded batches of a few items).
SMALL_BATCH_WORKLOADS = [k for k, w in WORKLOADS.items() if w.n <= 256]

# Dense workloads of the fused small-n syev: seeded symmetric matrices with
# a lower triangle of iid N(0,1) entries (random_symmetric), at the orders
# and batches the syev tables on the pages use for the small-n kernels.
DENSE_WORKLOADS: Dict[str, Tuple[str, int, int]] = {
    # name: (dtype, n, batch)
    "s_f32_n8": ("f32", 8, 65536),
    "s_f32_n16": ("f32", 16, 32768),
    "s_f32_n32": ("f32", 32, 16384),
    "s_f64_n16": ("f64", 16, 32768),
    "s_f64_n32": ("f64", 32, 16384),
}


def make_dense(name: str, batch: int | None = None) -> np.ndarray:
    """Dense (batch, n, n) matrices of a DENSE_WORKLOADS entry; a smaller
    batch is a prefix of the full one."""
    dt, n, nb = DENSE_WORKLOADS[name]
    nb = nb if batch is None else int(batch)
    return random_symmetric(n, nb, np.float32 if dt == "f32" else np.float64, cfg=9)


def rng_for(cfg: int, n: int, salt: int | None = None) -> np.random.Generator:
    """PCG64 generator seeded from (1234, cfg, n[, salt])."""
    key = [SEED, int(cfg), int(n)]
    if salt is not None:
        key.append(int(salt))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def edge_kind(b: int) -> int | None:
    """Edge kind of item b in a mixed batch, or None for an ordinary item.

    Item b with b mod 10 == 9 is an edge item of kind (b div 10) mod 5.
    """
    if b % 10 != 9:
        return None
    return (b // 10) % 5


def _apply_edge(kind: int, b: int, d: np.ndarray, e: np.ndarray) -> None:
    """Overwrite one item's (d, e) in place with the edge recipe of `kind`.

    d and e arrive holding an ordinary iid N(0,1) item; some recipes keep it
    (split, scaled, NaN) and some replace it (graded, zero).
    """
    n = d.shape[0]
    if kind == EDGE_SPLIT:
        for i in (n // 4 - 1, n // 2 - 1, 3 * n // 4 - 1):
            if 0 <= i < n - 1:
                e[i] = 0.0
    elif kind == EDGE_GRADED:
        # d_i = 10^(-i/2) up to order 64; longer items are graded over the
        # same 31.5 decades so that float32 entries stay normal numbers
        z = e.copy()
        step = 0.5 * min(1.0, 64.0 / n)
        d[:] = 10.0 ** (-np.arange(n, dtype=np.float64) * step)
        if n > 1:
            e[:] = z * np.sqrt(d[:-1] * d[1:])
    elif kind == EDGE_ZERO:
        d[:] = 0.0
        e[:] = 0.0
    elif kind == EDGE_SCALED:
        f = 1e18 if (b // 50) % 2 == 0 else 1e-18
        d *= f
        e *= f
    elif kind == EDGE_NAN:
        j = (7919 * b) % (2 * n - 1)
        if j < n:
            d[j] = np.nan
        else:
            e[j - n] = np.nan
    else:  # pragma: no cover - defensive
        raise ValueError(kind)


def make_batch(w: Workload, batch: int | None = None, dtype=None,
               replicate: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Return (d, e) for workload `w`.

    batch: number of items (default: the workload's own batch). The d rows
        of a smaller batch are the first rows of the full batch's; e is drawn
        after d, so its rows depend on the batch size (each (workload, batch)
        pair is one fixed seeded sample).
    dtype: numpy dtype of the result (default: the workload's dtype).
    replicate: if > 1, every item is repeated `replicate` times in a row
        (item k of the result is base item k // replicate). Used to measure
        the lockstep ideal, where every chunk of a wavefront holds the same
        problem.
    """
    nb = w.batch if batch is None else int(batch)
    base_nb = -(-nb // replicate)
    n = w.n
    g = rng_for(w.cfg, n)
    # d for the whole batch, then e (a fixed order of draws per batch size)
    d = g.standard_normal((base_nb, n))
    e = g.standard_normal((base_nb, max(n - 1, 0)))
    if w.edge_mix:
        for b in range(base_nb):
            k = edge_kind(b)
            if k is not None:
                _apply_edge(k, b, d[b], e[b])
    if replicate > 1:
        d = np.repeat(d, replicate, axis=0)[:nb]
        e = np.repeat(e, replicate, axis=0)[:nb]
    dt = w.np_dtype if dtype is None else dtype
    return np.ascontiguousarray(d.astype(dt)), np.ascontiguousarray(e.astype(dt))


def random_batch(n: int, batch: int, dtype=np.float64, salt: int = 0,
                 cfg: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """iid N(0,1) d and e for arbitrary (n, batch); used by sweeps over n."""
    g = rng_for(cfg, n, salt)
    d = g.standard_normal((batch, n))
    e = g.standard_normal((batch, max(n - 1, 0)))
    return (np.ascontiguousarray(d.astype(dtype)),
            np.ascontiguousarray(e.astype(dtype)))


def random_basis(n: int, batch: int, dtype=np.float64, salt: int = 0,
                 orthogonal: bool = True) -> np.ndarray:
    """Seeded (batch, n, n) row-major basis for back-transformation tests:
    the orthogonal factor of a Gaussian matrix (numpy QR in float64, then
    rounded to dtype), or with orthogonal=False the Gaussian matrix itself."""
    g = rng_for(7, n, salt)
    a = g.standard_normal((batch, n, n))
    if orthogonal and n > 0:
        a = np.linalg.qr(a)[0]
    return np.ascontiguousarray(a.astype(dtype))


def random_symmetric(n: int, batch: int, dtype=np.float64, salt: int = 0,
                     cfg: int = 8) -> np.ndarray:
    """Seeded dense symmetric (batch, n, n) row-major matrices: the lower
    triangle (diagonal included) iid N(0,1), mirrored into the upper one."""
    g = rng_for(cfg, n, salt)
    a = np.tril(g.standard_normal((batch, n, n)))
    a = a + np.swapaxes(np.tril(a, -1), 1, 2)
    return np.ascontiguousarray(a.astype(dtype))


def edge_batch(kind: int, n: int, batch: int, dtype=np.float64,
               salt: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """A batch made only of edge items of one kind (for the edge-case tests).

    Item b uses the same recipe as item b of a mixed batch would if it were
    an edge item of this kind (so scaled items alternate 1e18 / 1e-18 every
    50 items; here item b uses 1e18 when b is even, 1e-18 when odd, and NaN
    positions follow (7919*b) mod (2n-1)).
    """
    g = rng_for(100 + kind, n, salt)
    d = g.standard_normal((batch, n))
    e = g.standard_normal((batch, max(n - 1, 0)))
    for b in range(batch):
        bb = b * 50 if kind == EDGE_SCALED else b
        _apply_edge(kind, bb, d[b], e[b])
    return (np.ascontiguousarray(d.astype(dtype)),
            np.ascontiguousarray(e.astype(dtype)))


def toeplitz_batch(n: int, a: float, b: float, batch: int = 1,
                   dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """Constant-diagonal tridiagonal matrices tridiag(b; a; b)."""
    d = np.full((batch, n), a, dtype=np.float64)
    e = np.full((batch, max(n - 1, 0)), b, dtype=np.float64)
    return d.astype(dtype), e.astype(dtype)


def dense_from_bands(d: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Dense (batch, n, n) symmetric tridiagonal matrices from bands."""
    nb, n = d.shape
    T = np.zeros((nb, n, n), dtype=d.dtype)
    idx = np.arange(n)
    T[:, idx, idx] = d
    if n > 1:
        T[:, idx[:-1], idx[1:]] = e
        T[:, idx[1:], idx[:-1]] = e
    return T


def list_workloads() -> List[str]:
    return list(WORKLOADS)
