"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/steqr.h declares, plans launches, and rejects bad arguments
before touching the device (those paths make no HIP call)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "steqr.h")
LIB = os.path.join(ROOT, "symmetric_tridiagonal_eigensolver_amd", "libsteqr.so")


def _ensure_built():
    if not os.path.exists(LIB):
        import __graft_entry__ as g
        g.build()


@pytest.fixture(scope="module")
def st():
    _ensure_built()
    import symmetric_tridiagonal_eigensolver_amd as st
    return st


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:steqr|syev)_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared() == ["steqr_batched", "steqr_batched_ex", "steqr_query", "steqr_version",
                           "syev_batched", "syev_batched_ex", "syev_query"]


def test_library_exports_every_declared_symbol(st):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in _declared():
        assert name in exported, name
        assert hasattr(st.lib(), name)
    assert set(st.EXPORTS) == set(_declared())


def test_library_links_no_oracle():
    out = subprocess.run(["nm", "-D", LIB], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in out


def test_version(st):
    assert "gfx950" in st.version()


@pytest.mark.parametrize("dtype,jobz,n,cases", [
    (0, 1, 16, [(512, 16), (8192, 16), (16384, 8), (32767, 8), (32768, 4), (262144, 4)]),
    (0, 1, 8, [(1000, 8), (16384, 8), (32768, 4), (65535, 4), (65536, 2)]),
    (0, 1, 32, [(1000, 16), (16383, 16), (16384, 8), (32768, 8)]),
    (1, 1, 16, [(1000, 8), (16383, 8), (16384, 4), (32768, 4)]),
    (0, 0, 16, [(1000, 4), (16384, 4), (32768, 2), (65535, 2), (65536, 1), (262144, 1)]),
    (0, 0, 32, [(1000, 4), (32768, 4), (65536, 2), (131071, 2), (131072, 1)]),
    (1, 0, 32, [(1000, 2), (16384, 2), (32767, 2), (32768, 1)]),
    # outside the batch rule: fixed lanes at any batch
    (0, 1, 4, [(512, 4), (262144, 4)]), (1, 1, 12, [(512, 4), (262144, 4)]),
    (1, 1, 32, [(512, 16), (262144, 16)]), (0, 0, 8, [(512, 1), (262144, 1)]),
    (1, 0, 16, [(512, 1), (262144, 1)]),
    # order 128 values only in float; order 64 in double with eigenvectors
    # (producer lanes: 11 problems per workgroup at 4, 3 at 16)
    (0, 0, 128, [(256, 16), (8192, 16), (16383, 16), (16384, 8)]),
    (1, 0, 128, [(256, 16), (65536, 16)]),
    (1, 1, 64, [(256, 16), (2815, 16), (2816, 4), (16384, 4)]),
    (0, 1, 64, [(256, 16), (16384, 16)]),
    # order 64 without eigenvectors (producer lanes 4, 8, 16); order 128 in
    # float with eigenvectors (whole rows at 8, half rows at 32)
    (0, 0, 64, [(1024, 16), (16383, 16), (16384, 8), (32767, 8), (32768, 4)]),
    (1, 0, 64, [(4096, 16), (16384, 8), (65536, 4)]),
    (0, 1, 128, [(64, 32), (512, 32), (513, 8), (8192, 8)])])
def test_query_lanes_follow_batch(st, dtype, jobz, n, cases):
    """Orders 8..32 in their default band storage: the default lanes per
    problem are the fewest whose launch still has the case's wavefront
    count (2,048 in float with eigenvectors, 1,024 in double with them and
    in float values only at order 16, 2,048 at order 32, 512 in double
    values only at order 32), else the most of the case's candidates; an
    explicit band storage keeps the fixed choice."""
    for batch, P in cases:
        q = st.steqr_query(n, batch, jobz, dtype)
        assert q["lanes_per_problem"] == P, (batch, q)
    if dtype == 0 and n in (16, 32) and not jobz:
        q = st.steqr_query(n, 262144, 0, 0, st.make_params(band_storage=1))
        assert q["lanes_per_problem"] == 1
    if dtype == 0 and n == 16 and jobz:
        q = st.steqr_query(n, 512, 1, 0, st.make_params(band_storage=2))
        assert (q["lanes_per_problem"], q["band_storage"]) == (4, 2)


@pytest.mark.parametrize("n,jobz,dtype,N,P", [
    (1, 1, 0, 4, 4), (4, 1, 0, 4, 4), (5, 1, 0, 8, 4), (8, 0, 0, 8, 1), (12, 1, 1, 12, 4), (12, 0, 1, 16, 1),
    (16, 1, 0, 16, 4), (17, 1, 0, 32, 8), (32, 1, 1, 32, 16), (32, 0, 1, 32, 1), (32, 0, 0, 32, 4), (16, 0, 0, 16, 2), (16, 0, 1, 16, 1),
    (33, 1, 1, 64, 4), (64, 1, 1, 64, 4), (64, 1, 0, 64, 16), (64, 0, 0, 64, 4),
    (40, 0, 1, 64, 4), (100, 1, 0, 128, 8), (100, 1, 1, 128, 32), (128, 0, 0, 128, 8),
    (128, 0, 1, 128, 16),
    (129, 1, 0, 256, 64), (256, 1, 1, 256, 64), (200, 0, 0, 256, 64), (256, 0, 1, 256, 64),
    (257, 1, 0, 512, 64), (512, 1, 1, 512, 64), (300, 0, 0, 512, 64), (512, 0, 1, 512, 64)])
def test_query_default_plan(st, n, jobz, dtype, N, P):
    """Default launches at the configurations' batch of 32,768 (orders
    8..32 pick their lanes by batch: test_query_lanes_follow_batch)."""
    B = 32768
    q = st.steqr_query(n, B, jobz, dtype)
    assert q["padded_n"] == N and q["lanes_per_problem"] == P
    if q["band_storage"] == 3:
        # producer and consumer wavefronts: one problem per consumer
        assert n > 32 and jobz and q["rows_per_lane"] == 1
        # consumers per problem: 1 up to order 64; at 128 two (float, whole
        # rows) or four (double, half rows); at 256 eight (float, half rows:
        # one workgroup per problem) or sixteen (double, quarter rows: two
        # workgroups per problem); at 512 sixty-four (float, eighth rows:
        # eight workgroups per problem) or 128 (double, sixteenth rows:
        # sixteen workgroups per problem)
        if N >= 256:
            assert q["waves_per_block"] == 9
            gpp = {(256, 0): 1, (256, 1): 2, (512, 0): 8, (512, 1): 16}[(N, dtype)]
            assert q["workgroups"] == B * gpp
            return
        cpp = 1 if N <= 64 else (2 if dtype == 0 else 4)
        per_block = (q["waves_per_block"] - 1) // cpp
    else:
        assert q["rows_per_lane"] == ((N + P - 1) // P if jobz else 0)
        per_block = q["waves_per_block"] * (64 // P)
    assert q["workgroups"] == -(-B // per_block)


def test_query_producer_consumer_plans(st):
    """Orders 33..64 with eigenvectors default to producer and consumer
    wavefronts; band storage 2 still selects one problem per wavefront, and
    band 3 is rejected where no such kernel exists."""
    for dtype, w in ((0, 3), (1, 11)):
        q = st.steqr_query(50, 7000, 1, dtype)
        assert q["band_storage"] == 3 and q["waves_per_block"] == w + 1
        assert q["workgroups"] == -(-7000 // w)
        if dtype == 0:
            q2 = st.steqr_query(50, 700, 1, dtype, st.make_params(band_storage=2))
            assert q2["band_storage"] == 2 and q2["lanes_per_problem"] == 64
        else:
            # one problem per wavefront in double with eigenvectors needs
            # more than 256 registers per lane: not built
            with pytest.raises(st.SteqrError):
                st.steqr_query(50, 700, 1, dtype, st.make_params(band_storage=2))
        q3 = st.steqr_query(50, 700, 1, dtype, st.make_params(band_storage=1))
        assert q3["band_storage"] == 3
    for n, jobz in ((50, 0), (16, 1), (32, 1)):
        with pytest.raises(st.SteqrError):
            st.steqr_query(n, 100, jobz, 1, st.make_params(band_storage=3))


def test_query_explicit_lanes(st):
    prm = st.make_params(lanes_per_problem=4)
    q = st.steqr_query(16, 32768, 1, 0, prm)
    assert q["lanes_per_problem"] == 4 and q["rows_per_lane"] == 4
    assert 1 <= q["waves_per_block"] <= 4
    assert q["workgroups"] == 32768 // (q["waves_per_block"] * 16)
    q1 = st.steqr_query(16, 32768, 1, 0, st.make_params(lanes_per_problem=4, waves_per_block=1))
    assert q1["waves_per_block"] == 1 and q1["workgroups"] == 32768 // 16


@pytest.mark.parametrize("batch,waves", [(32768, 4), (4096, 1), (8192, 2), (1000, 1), (16384, 4)])
def test_query_small_batch_spreads_workgroups(st, batch, waves):
    # order 4 with eigenvectors: 16 problems per wavefront; the default packs
    # 4 wavefronts per workgroup unless that leaves fewer than 256 workgroups
    q = st.steqr_query(4, batch, 1, 0)
    assert q["waves_per_block"] == waves
    assert q["workgroups"] == -(-batch // (waves * 16))
    # an explicit choice is kept
    q4 = st.steqr_query(4, batch, 1, 0, st.make_params(waves_per_block=4))
    assert q4["waves_per_block"] == 4


def test_query_band_storage(st):
    assert st.steqr_query(16, 100, 1, 0)["band_storage"] == 1
    assert st.steqr_query(16, 100, 1, 1)["band_storage"] == 2
    assert st.steqr_query(32, 100, 1, 0)["band_storage"] == 2
    assert st.steqr_query(16, 100, 1, 0, st.make_params(band_storage=2))["band_storage"] == 2
    # orders above 32 always keep the band in LDS (with eigenvectors: the
    # producer and consumer wavefronts)
    assert st.steqr_query(40, 100, 1, 1, st.make_params(band_storage=1))["band_storage"] == 3
    assert st.steqr_query(40, 100, 0, 1, st.make_params(band_storage=1))["band_storage"] == 2
    with pytest.raises(st.SteqrError):
        st.steqr_query(16, 100, 1, 0, st.make_params(band_storage=4))


@pytest.mark.parametrize("args,rc", [
    # (d, e, lam, Q, n, batch, jobz, dtype) -> code
    ((0, 8, 8, 8, 4, 10, 1, 0), -1),
    ((8, 0, 8, 8, 4, 10, 1, 0), -2),
    ((8, 0, 8, 8, 1, 10, 1, 0), None),   # n == 1 needs no e: would launch, skipped
    ((8, 8, 0, 8, 4, 10, 1, 0), -3),
    ((8, 8, 8, 0, 4, 10, 1, 0), -4),
    ((8, 8, 8, 8, -1, 10, 1, 0), -5),
    ((8, 8, 8, 8, 513, 10, 1, 0), -5),
    ((8, 8, 8, 8, 4, -1, 1, 0), -6),
    ((8, 8, 8, 8, 4, 10, 2, 0), -7),
    ((8, 8, 8, 8, 4, 10, 1, 5), -8),
    # the first invalid argument in parameter order wins
    ((0, 8, 8, 8, 4, 10, 2, 0), -1),     # NULL d before a bad jobz
    ((8, 8, 0, 8, 4, 10, 1, 7), -3),     # NULL lambda before a bad dtype
    ((8, 8, 8, 0, 200, 10, 1, 0), -4),   # NULL Q before an unsupported n
    ((0, 8, 8, 8, -1, 10, 1, 0), -5),    # no work (n < 0): NULL d is not an error
    ((0, 0, 0, 0, 0, 10, 1, 0), 0),      # n == 0: quick return
    ((0, 0, 0, 0, 4, 0, 1, 0), 0),       # batch == 0: quick return
])
def test_argument_errors(st, args, rc):
    if rc is None:
        pytest.skip("valid call: would launch a kernel")
    d, e, lam, Q, n, batch, jobz, dtype = args
    got = st.lib().steqr_batched(d or None, e or None, lam or None, Q or None, n, batch,
                                 jobz, dtype, None)
    assert got == rc


def test_bad_params(st):
    # every call here is rejected by argument validation before any launch
    # (the pointers are not device memory)
    L = st.lib()
    for prm in (st.make_params(lanes_per_problem=3), st.make_params(lanes_per_problem=128),
                st.make_params(waves_per_block=3), st.make_params(lanes_per_problem=-4),
                st.make_params(update_scheme=2), st.make_params(update_scheme=-1),
                st.make_params(shift=2), st.make_params(shift=-1)):
        got = L.steqr_batched_ex(8, 8, 8, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm))
        assert got == -10
    for bt in (2, -1):
        prm = st.make_params()
        prm.back_transform = bt
        assert L.steqr_batched_ex(8, 8, 8, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm)) == -10
    # a NULL array is reported before a bad params field
    prm = st.make_params(lanes_per_problem=3)
    assert L.steqr_batched_ex(8, 8, None, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm)) == -3
    assert L.steqr_batched_ex(None, 8, 8, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm)) == -1
    # back-transformation needs eigenvectors
    prm = st.make_params(back_transform=True)
    assert L.steqr_batched_ex(8, 8, 8, 8, 16, 10, 0, 0, None, None, ctypes.byref(prm)) == -10
    with pytest.raises(st.SteqrError):
        st.steqr_query(16, 10, 0, 0, prm)
    assert st.steqr_query(16, 10, 1, 0, prm) == st.steqr_query(16, 10, 1, 0)


@pytest.mark.parametrize("n,jobz,dtype", [(4, 1, 0), (16, 1, 0), (16, 0, 0), (12, 1, 1),
                                          (32, 1, 0), (32, 0, 1), (64, 1, 1), (50, 0, 0)])
def test_pg_scheme_has_the_same_plans(st, n, jobz, dtype):
    """Every launch plan exists in both forms of the chase step."""
    for lanes in (0, 1, 2, 4, 8, 16, 32, 64):
        for band in (0, 1, 2):
            try:
                a = st.steqr_query(n, 1000, jobz, dtype,
                                   st.make_params(lanes_per_problem=lanes, band_storage=band))
            except st.SteqrError:
                with pytest.raises(st.SteqrError):
                    st.steqr_query(n, 1000, jobz, dtype,
                                   st.make_params(lanes_per_problem=lanes, band_storage=band,
                                                  update_scheme=st.STEQR_PG))
                continue
            b = st.steqr_query(n, 1000, jobz, dtype,
                               st.make_params(lanes_per_problem=lanes, band_storage=band,
                                              update_scheme=st.STEQR_PG))
            assert a == b


def test_uninstantiated_lanes_rejected_by_query(st):
    with pytest.raises(st.SteqrError) as ex:
        st.steqr_query(16, 10, 1, 0, st.make_params(lanes_per_problem=64))
    assert ex.value.rc == -10


# ---------------------------------------------------------------- dense syev

@pytest.mark.parametrize("n,jobz,dtype,N,P,R", [
    (1, 1, 0, 4, 4, 1), (4, 1, 0, 4, 4, 1), (5, 1, 0, 8, 4, 2), (16, 1, 0, 16, 4, 4),
    (16, 0, 0, 16, 4, 4), (12, 1, 1, 16, 8, 2), (17, 1, 0, 32, 16, 2), (32, 0, 1, 32, 32, 1),
    (8, 0, 1, 8, 4, 2), (32, 0, 0, 32, 8, 4), (16, 0, 1, 16, 4, 4), (16, 1, 1, 16, 8, 2),
    (32, 1, 1, 32, 32, 1), (20, 1, 1, 32, 32, 1)])
def test_syev_default_plans(st, n, jobz, dtype, N, P, R):
    q = st.syev_query(n, 32768, jobz, dtype)
    assert (q["padded_n"], q["lanes_per_problem"], q["rows_per_lane"]) == (N, P, R)
    # the band in registers except for double at order 32
    assert q["band_storage"] == (2 if (dtype, N) == (1, 32) else 1)
    per_block = q["waves_per_block"] * 64 // P
    assert q["workgroups"] == -(-32768 // per_block)


@pytest.mark.parametrize("n,jobz,dtype,cases", [
    (8, 1, 0, [(1024, 4), (32767, 4), (32768, 4), (65536, 2)]),
    (16, 1, 0, [(1024, 8), (16384, 8), (32768, 4), (65536, 4)]),
    (32, 0, 0, [(1024, 16), (16383, 16), (16384, 8)]),
    (16, 0, 1, [(1024, 8), (16383, 8), (16384, 4), (32768, 4)]),
    (16, 0, 0, [(1024, 4), (65536, 4)]), (8, 0, 0, [(1024, 2), (65536, 2)])])
def test_syev_lanes_follow_batch(st, n, jobz, dtype, cases):
    """The fused dense solver's default lanes per problem: more lanes for
    batches that would leave SIMDs idle (the tuned choice at the
    configurations' batches)."""
    for batch, P in cases:
        assert st.syev_query(n, batch, jobz, dtype)["lanes_per_problem"] == P, batch


def test_syev_argument_errors(st):
    L = st.lib()
    # validation happens before any launch (the pointers are not device memory)
    assert L.syev_batched(8, 8, 8, 33, 10, 1, 0, None) == -4
    assert L.syev_batched(8, 8, 8, 33, 10, 1, 1, None) == -4   # double with vectors: n <= 32
    assert L.syev_batched(8, 8, 8, -1, 10, 1, 0, None) == -4
    assert L.syev_batched(8, 8, 8, 16, -1, 1, 0, None) == -5
    assert L.syev_batched(8, 8, 8, 16, 10, 2, 0, None) == -6
    assert L.syev_batched(8, 8, 8, 16, 10, 1, 2, None) == -7
    assert L.syev_batched(None, 8, 8, 16, 10, 1, 0, None) == -1
    assert L.syev_batched(8, None, 8, 16, 10, 1, 0, None) == -2
    assert L.syev_batched(8, 8, None, 16, 10, 1, 0, None) == -3
    assert L.syev_batched(None, 8, 8, 16, 10, 2, 0, None) == -1   # NULL A before a bad jobz
    assert L.syev_batched(8, None, 8, 40, 10, 1, 0, None) == -2   # NULL lambda before n
    assert L.syev_batched(None, None, None, 0, 10, 1, 0, None) == 0
    assert L.syev_batched(None, None, None, 16, 0, 1, 0, None) == 0
    for prm in (st.make_params(update_scheme=st.STEQR_PG), st.make_params(back_transform=True),
                st.make_params(band_storage=2), st.make_params(lanes_per_problem=64),
                st.make_params(waves_per_block=3), st.make_params(shift=2)):
        assert L.syev_batched_ex(8, 8, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm)) == -10
    # band storage: 1 or 2 where that variant is built
    p1, p2, p3 = (st.make_params(band_storage=b) for b in (1, 2, 3))
    assert L.syev_batched_ex(8, 8, 8, 32, 10, 1, 1, None, None, ctypes.byref(p1)) == -10
    assert L.syev_batched_ex(8, 8, 8, 32, 10, 1, 1, None, None, ctypes.byref(p3)) == -10
    assert st.syev_query(32, 10, 1, 1, p2)["band_storage"] == 2
    assert st.syev_query(16, 10, 1, 0, p1)["band_storage"] == 1
    assert st.syev_query(32, 10, 0, 1, p1)["band_storage"] == 1
    # the closed-form shift is accepted
    assert st.syev_query(16, 10, 1, 0, st.make_params(shift=st.STEQR_SHIFT_CLOSED))["padded_n"] == 16


# ---------------------------------------------------------------- bisection

@pytest.mark.parametrize("n,dtype,N,band", [(1, 0, 4, 1), (3, 1, 4, 1), (16, 0, 16, 1),
                                            (17, 1, 32, 1), (64, 0, 64, 1), (40, 1, 64, 2),
                                            (65, 0, 128, 2), (128, 1, 128, 2), (129, 0, 256, 2),
                                            (256, 1, 256, 2), (257, 0, 512, 2), (512, 1, 512, 2)])
def test_bisect_plans(st, n, dtype, N, band):
    q = st.steqr_query(n, 32768, 0, dtype, st.make_params(method=st.STEQR_METHOD_BISECT))
    L = min(N, 64)
    assert (q["padded_n"], q["lanes_per_problem"], q["rows_per_lane"], q["band_storage"]) == \
        (N, L, 0, band)
    assert q["workgroups"] == -(-32768 // (q["waves_per_block"] * 64 // L))


@pytest.mark.parametrize("n,dtype,batch,P,waves,wgs", [
    (512, 0, 256, 256, 4, 256), (512, 1, 1024, 128, 2, 1024), (512, 0, 2048, 64, 4, 512),
    (300, 1, 2047, 128, 2, 2047), (256, 0, 1024, 128, 2, 1024), (256, 1, 4096, 64, 4, 1024),
    (200, 0, 100, 256, 4, 100), (128, 0, 8192, 64, 4, 2048), (128, 1, 1000, 128, 2, 1000),
    (100, 0, 10, 128, 2, 10), (64, 0, 10, 64, 4, 3)])
def test_bisect_wavefronts_per_problem(st, n, dtype, batch, P, waves, wgs):
    """From order 128 the bisection spreads a problem's eigenvalue indices
    over 1, 2 or 4 wavefronts of one workgroup (64, 128 or 256 lanes per
    problem): the fewest whose launch has 2,048 wavefronts."""
    q = st.steqr_query(n, batch, 0, dtype, st.make_params(method=st.STEQR_METHOD_BISECT))
    assert (q["lanes_per_problem"], q["waves_per_block"], q["workgroups"]) == (P, waves, wgs)


def test_bisect_lanes_choices(st):
    def q(n, lanes):
        return st.steqr_query(n, 100, 0, 0, st.make_params(method=1, lanes_per_problem=lanes))
    for n, lanes, waves in ((512, 64, 4), (512, 128, 2), (512, 256, 4), (256, 256, 4),
                            (128, 128, 2), (64, 64, 4), (16, 16, 4)):
        r = q(n, lanes)
        assert (r["lanes_per_problem"], r["waves_per_block"]) == (lanes, waves)
    # more lanes than the padded order, eight wavefronts, fewer than a
    # wavefront from order 64, or more than one below order 128: rejected
    for n, lanes in ((128, 256), (512, 512), (512, 32), (64, 128), (100, 32), (16, 64)):
        with pytest.raises(st.SteqrError):
            q(n, lanes)


def test_bisect_argument_errors(st):
    L = st.lib()
    bad = [st.make_params(method=2), st.make_params(method=-1),
           st.make_params(method=1, update_scheme=st.STEQR_PG),
           st.make_params(method=1, shift=1), st.make_params(method=1, band_storage=2),
           st.make_params(method=1, lanes_per_problem=4)]
    for prm in bad:
        assert L.steqr_batched_ex(8, 8, 8, 8, 16, 10, 0, 0, None, None, ctypes.byref(prm)) == -10
    # values only
    prm = st.make_params(method=1)
    assert L.steqr_batched_ex(8, 8, 8, 8, 16, 10, 1, 0, None, None, ctypes.byref(prm)) == -10
    # the padded order as lanes is accepted
    assert st.steqr_query(12, 10, 0, 0, st.make_params(method=1, lanes_per_problem=16))["padded_n"] == 16
    # syev does not take the bisection method
    assert L.syev_batched_ex(8, 8, 8, 16, 10, 0, 0, None, None, ctypes.byref(prm)) == -10


def _case_lists():
    """The (dtype, n, jobz, lanes, band, scheme) launches the GPU tests make."""
    import test_gpu_back_transform as BT
    import test_gpu_big as BIG
    import test_gpu_parity as GP
    import test_gpu_pg as PGT
    out = []
    for c in GP.LANE_CASES:
        if hasattr(c, "values"):  # a skipped pytest.param: not launched
            continue
        dt, n, jobz, lanes, band = c
        out.append((dt, n, jobz, lanes, band, 0))
    for dt, n, jobz, lanes, band in PGT.PG_LANES:
        out.append((dt, n, jobz, lanes, band, 1))
    for dt, n, lanes, band in BT.KERNEL_CASES:
        out += [(dt, n, True, lanes, band, 0), (dt, n, True, lanes, band, 1)]
    for mark in BIG.test_big_producer_shapes.pytestmark:
        if mark.name == "parametrize":
            out += [(dt, n, True, lanes, 0, 0) for dt, lanes in mark.args[1] for n in (80, 128)]
    for dt in (np.float32, np.float64):
        for jobz in (True, False):
            out += [(dt, n, jobz, 0, 0, sc) for n in (129, 200, 256) for sc in (0, 1)]
            out += [(dt, n, jobz, 0, 0, sc) for n in (257, 450, 512) for sc in (0, 1)]
        out += [(dt, 240, False, 16, 0, 0)]
    for dt in (np.float32, np.float64):
        for band in (1, 2):
            for n in ((9, 16) if (dt == np.float64 and band == 1) else (9, 16, 32)):
                out.append((dt, n, True, 0, band, 0))
    return out


def test_gpu_test_cases_have_built_kernels(st):
    """Every launch shape the GPU tests request has a built kernel (no
    GPU needed: steqr_query plans without launching)."""
    for dt, n, jobz, lanes, band, scheme in _case_lists():
        code = st.STEQR_F32 if dt == np.float32 else st.STEQR_F64
        st.steqr_query(n, 777, int(jobz), code,
                       st.make_params(lanes_per_problem=lanes, band_storage=band,
                                      update_scheme=scheme))


def test_syev_test_cases_have_built_kernels(st):
    import test_gpu_syev as SY
    for dt, n, lanes, jobz in SY.CASES:
        code = st.STEQR_F32 if dt == np.float32 else st.STEQR_F64
        st.syev_query(n, 777, int(jobz), code, st.make_params(lanes_per_problem=lanes))


def test_c_caller_compiles_against_the_header(tmp_path):
    """include/steqr.h is valid C: the plain C caller of the ABI compiles and
    links against libsteqr.so (it runs in tests/test_gpu_c_abi.py)."""
    import shutil
    import subprocess
    import __graft_entry__ as g
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    out = str(tmp_path / "steqr_c_check")
    r = subprocess.run(g.c_check_command(out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert os.path.exists(out)
