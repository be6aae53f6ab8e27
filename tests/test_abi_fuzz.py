"""Randomised checks of the C ABI's argument validation (CPU only: without a GPU a
call that passes every check fails at its launch with MOE_ELAUNCH, so no kernel
runs on the stand-in pointers).  A model of the rules stated in
include/moe_expert.h predicts each call's status: MOE_EINVAL for an argument out
of range, NULL or misaligned, MOE_ENOTSUP for an unimplemented option, else the
launch.  Draws concentrate on the limits (H around 1024 / 8192 and off the
32-grid, K around 16, instance counts around 1024, pointer offsets up to 12)."""
import math

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests.test_abi import P, _no_gpu, combine, dispatch, gemm

pytestmark = pytest.mark.skipif(not _no_gpu(),
                                reason="valid calls would launch on stand-in pointers")

EINVAL, ENOTSUP, ELAUNCH = 1, 2, 3
SETTINGS = settings(max_examples=400, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])

bs = st.sampled_from([-1, 0, 1, 2, 511, 512, 513])
ks = st.sampled_from([-1, 0, 1, 8, 15, 16, 17])
hs = st.sampled_from([0, 992, 1000, 1024, 1056, 4096, 7168, 7184, 8192, 8224, 16384])
offs = st.sampled_from([0, 0, 0, 1, 2, 4, 8, 12])   # pointer misalignment in bytes


def ptr(off, null=False):
    return None if null else P + off


@SETTINGS
@given(Bs=bs, H=hs, K=ks, eps=st.sampled_from([0.0, 1e-6, -1e-6, math.inf, math.nan, 1.0]),
       mode=st.sampled_from([-1, 0, 1, 2]),
       o=st.lists(offs, min_size=10, max_size=10),
       null=st.lists(st.booleans(), min_size=9, max_size=9).map(
           lambda v: [b and (i % 3 == 0) for i, b in enumerate(v)]))
def test_combine_validation(Bs, H, K, eps, mode, o, null):
    names = ["eo", "asg", "s", "sh", "res", "g", "y", "xo", "rstd", "err"]
    optional = {"sh", "xo", "rstd", "err"}
    align = {"eo": 16, "asg": 4, "s": 4, "sh": 16, "res": 16, "g": 16, "y": 16, "xo": 16,
             "rstd": 4, "err": 4}
    isnull = dict(zip(names, null + [False]))
    kw = {n: ptr(o[j], isnull[n]) for j, n in enumerate(names)}
    expect = ELAUNCH
    if any(isnull[n] for n in names if n not in optional):
        expect = EINVAL
    elif not (0 < Bs <= 512 and 0 < K <= 16 and 1024 <= H <= 8192 and H % 32 == 0):
        expect = EINVAL
    elif not (eps >= 0 and math.isfinite(eps)) or mode not in (0, 1):
        expect = EINVAL
    elif any(not isnull[n] and o[j] % align[n] for j, n in enumerate(names)):
        expect = EINVAL
    assert combine(Bs=Bs, H=H, K=K, eps=eps, mode=mode, **kw) == expect


@SETTINGS
@given(Bs=bs, H=hs, K=ks, R=st.sampled_from([0, 1, 2, 32, 64, 65]),
       L=st.sampled_from([0, 1, 8, 16, 17]), q=st.sampled_from([-1, 0, 1, 2, 3, 4, 5, 6, 7]),
       tile=st.sampled_from([-1, 0, 8, 16, 96, 128, 1024, 2048]),
       qk=st.sampled_from([-1, 0, 1, 2, 3, 4]), qs_null=st.booleans(), sc_null=st.booleans(),
       o=st.lists(offs, min_size=10, max_size=10))
def test_dispatch_validation(Bs, H, K, R, L, q, tile, qk, qs_null, sc_null, o):
    x, ids, ex, cnt, off, src, asg, qs, sc, mask = o
    E = R * L
    expect = ELAUNCH
    if not (0 < Bs <= 512 and 0 < K <= 16 and 1024 <= H <= 8192 and H % 32 == 0):
        expect = EINVAL
    elif R < 1 or L < 1 or E > 1024 or K > E:
        expect = EINVAL
    elif qk < 0 or qk > 3 or (qk == 0) != qs_null:
        expect = EINVAL
    elif not qs_null and qs % (16 if qk in (2, 3) else 4):
        expect = EINVAL
    elif q not in (0, 1, 2, 3, 4, 5, 6):
        expect = EINVAL
    elif ((q in (0, 4, 5) and qk != 0) or (q == 1 and qk == 0) or (q == 6 and qk != 1) or
          (q in (2, 3) and qk not in (0, 3))):
        expect = EINVAL
    elif q in (2, 3, 4, 5) and sc_null:
        expect = EINVAL
    elif q == 3 and tile <= 0:
        expect = EINVAL
    elif q == 3 and (tile < 16 or tile > 1024 or tile & (tile - 1)):
        expect = ENOTSUP
    elif x % 16 or ex % 16 or ids % 16 or cnt % 4 or off % 4 or src % 4 or asg % 4:
        expect = EINVAL
    elif q in (2, 3) and not sc_null and sc % 4:
        expect = EINVAL
    elif mask % 4:
        expect = EINVAL
    got = dispatch(Bs=Bs, H=H, K=K, R=R, L=L, q=q, tile=tile, qs=ptr(qs, qs_null), qk=qk,
                   x=ptr(x), ids=ptr(ids), ex=ptr(ex), cnt=ptr(cnt), off=ptr(off),
                   src=ptr(src), asg=ptr(asg), sc=ptr(sc, sc_null), mask=ptr(mask))
    assert got == expect


@SETTINGS
@given(E=st.sampled_from([0, 1, 8, 1024, 1025]),
       rows=st.sampled_from([-1, 0, 1, 4096, 1 << 22, (1 << 22) + 1]),
       N=st.sampled_from([0, 100, 128, 4096, 16384, 16512]),
       H=st.sampled_from([0, 128, 7168, 7200, 16384, 16512]),
       q=st.sampled_from([-1, 0, 1, 2, 3, 4, 5, 6, 7]),
       o=st.lists(offs, min_size=7, max_size=7))
def test_gemm_validation(E, rows, N, H, q, o):
    a, asc, off, w, wsc, y, err = o
    expect = ELAUNCH
    if not (1 <= E <= 1024 and 0 <= rows <= (1 << 22)):
        expect = EINVAL
    elif not (128 <= H <= 16384 and H % 128 == 0 and 128 <= N <= 16384 and N % 128 == 0):
        expect = EINVAL
    elif q < 0 or q > 6:
        expect = EINVAL
    elif q not in (2, 3, 4, 5):
        expect = ENOTSUP
    elif a % 16 or w % 16 or y % 16 or asc % 4 or wsc % 4 or off % 4 or err % 4:
        expect = EINVAL
    got = gemm(a=ptr(a), asc=ptr(asc), off=ptr(off), E=E, rows=rows, w=ptr(w), wsc=ptr(wsc),
               N=N, H=H, q=q, y=ptr(y), err=ptr(err))
    assert got == expect


@SETTINGS
@given(Bs=bs, K=ks, nl=st.sampled_from([0, 1, 16, 512, 1024, 1025]),
       F=st.sampled_from([0, 1, 2, 3, 513, 1025, 1026]),
       ni=st.sampled_from([0, 1, 256, 1024, 1025]), sc_given=st.booleans(),
       thr_given=st.booleans(), o=st.lists(offs, min_size=6, max_size=6))
def test_update_expert_validation(Bs, K, nl, F, ni, sc_given, thr_given, o):
    from tests.test_abi import update
    ids, tab, oi, sc, thr, err = o
    expect = ELAUNCH
    if not (0 < Bs <= 512 and 0 < K <= 16) or nl <= 0 or nl > 1024 or K > nl:
        expect = EINVAL
    elif F < 2 or F > nl + 1 or ni <= 0 or ni > 1024:
        expect = EINVAL
    elif (ids % 4 or tab % 4 or oi % 4 or (sc_given and sc % 4) or (thr_given and thr % 4)
          or err % 4):
        expect = EINVAL
    got = update(ids=ptr(ids), t=ptr(tab), oi=ptr(oi), sc=ptr(sc, not sc_given),
                 thr=ptr(thr, not thr_given), err=ptr(err), Bs=Bs, K=K, nl=nl, F=F, ni=ni)
    assert got == expect
