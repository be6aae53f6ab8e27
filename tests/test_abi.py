"""The C ABI without a GPU: the library loads, exports every function that
include/moe_expert.h declares, and rejects out-of-range arguments on the
host before anything is enqueued.

Only calls that must fail validation are made here (no buffer is ever
touched), and only when no GPU is visible: a validation bug then shows up as
a launch error, never as a kernel running on made-up pointers.
"""
import ctypes as C
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_expert.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["moe_combine_add_rmsnorm", "moe_dispatch",
                                    "moe_expert_gemm", "moe_expert_swiglu", "moe_status_string",
                                    "moe_update_dispatch", "moe_update_expert"]


def test_library_exports_every_declared_symbol():
    from combine_expert_amd import moe
    lib = C.CDLL(moe.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.library_path()], capture_output=True,
                         text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_status_strings():
    from combine_expert_amd import moe
    assert moe.moe_status_string(0).startswith("MOE_OK")
    assert moe.moe_status_string(1).startswith("MOE_EINVAL")
    assert moe.moe_status_string(2).startswith("MOE_ENOTSUP")
    assert moe.moe_status_string(3).startswith("MOE_ELAUNCH")
    assert moe.moe_status_string(42) == "unknown moe_status"


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced by these calls


def dispatch(**kw):
    from combine_expert_amd import moe
    a = dict(x=P, ids=P, mask=None, Bs=512, H=7168, K=8, R=32, L=8, q=4, tile=0, qs=None, qk=0,
             ex=P, sc=P, cnt=P, off=P, src=P, asg=P, err=None)
    a.update(kw)
    return moe.raw().moe_dispatch(a["x"], a["ids"], a["mask"], None, a["Bs"], a["H"], a["K"],
                                  a["R"],
                                  a["L"], a["q"], a["tile"], a["qs"], a["qk"], a["ex"], a["sc"],
                                  a["cnt"], a["off"], a["src"], a["asg"], a["err"], None)


def combine(**kw):
    from combine_expert_amd import moe
    a = dict(eo=P, asg=P, s=P, sh=None, res=P, g=P, eps=1e-6, Bs=512, H=7168, K=8, mode=0,
             y=P, xo=None, rstd=None, err=None)
    a.update(kw)
    return moe.raw().moe_combine_add_rmsnorm(a["eo"], a["asg"], a["s"], a["sh"], a["res"],
                                             a["g"], a["eps"], a["Bs"], a["H"], a["K"],
                                             a["mode"], a["y"], a["xo"], a["rstd"], a["err"],
                                             None)


def update(**kw):
    from combine_expert_amd import moe
    a = dict(ids=P, sc=None, t=P, thr=None, tm=None, Bs=512, K=16, nl=512, F=3, ni=1024,
             oi=P, om=P, err=None)
    a.update(kw)
    return moe.raw().moe_update_expert(a["ids"], a["sc"], a["t"], a["thr"], a["tm"], a["Bs"],
                                       a["K"], a["nl"], a["F"], a["ni"], a["oi"], a["om"],
                                       a["err"], None)


def limits():
    with open(os.path.join(ROOT, "tests", "golden", "page_constraints.json")) as f:
        return json.load(f)


@pytest.mark.skipif("not _no_gpu()")
def test_dispatch_rejects_out_of_range_arguments():
    g = limits()["combine_shapes"]
    bad = [dict(Bs=0), dict(Bs=g["Bs"]["max"] + 1), dict(K=0), dict(K=g["K"]["max"] + 1),
           dict(H=g["H"]["min"] - 32), dict(H=g["H"]["max"] + 32), dict(H=7168 + 16),
           dict(R=0), dict(L=0), dict(R=64, L=17), dict(R=1, L=4, K=8), dict(q=7), dict(q=-1),
           dict(x=None), dict(ids=None), dict(ex=None), dict(cnt=None), dict(off=None),
           dict(src=None), dict(asg=None), dict(q=2, sc=None), dict(q=4, sc=None),
           dict(q=5, sc=None), dict(q=5, qs=P, qk=1),
           dict(q=3, tile=128, sc=None), dict(q=3, tile=0), dict(x=P + 8), dict(ex=P + 4),
           dict(ids=P + 4), dict(q=2, sc=P + 2), dict(mask=P + 1),
           # the scales input: shape named iff present, a shape the mode takes, aligned
           dict(q=1), dict(q=1, qk=1), dict(q=1, qs=P), dict(q=1, qs=P, qk=4),
           dict(q=1, qs=P, qk=-1), dict(q=0, qs=P, qk=1), dict(q=4, qs=P, qk=3),
           dict(q=2, qs=P, qk=1), dict(q=2, qs=P, qk=2), dict(q=3, tile=128, qs=P, qk=2),
           dict(q=1, qs=P + 4, qk=2), dict(q=2, qs=P + 8, qk=3), dict(q=1, qs=P + 2, qk=1),
           # the second static type takes one coefficient only
           dict(q=6), dict(q=6, qs=P, qk=2), dict(q=6, qs=P, qk=3), dict(q=6, qs=P + 2, qk=1)]
    for kw in bad:
        assert dispatch(**kw) == 1, kw
    for kw in (dict(q=3, tile=96), dict(q=3, tile=8), dict(q=3, tile=2048)):
        assert dispatch(**kw) == 2, kw


@pytest.mark.skipif("not _no_gpu()")
def test_combine_rejects_out_of_range_arguments():
    bad = [dict(Bs=0), dict(Bs=513), dict(K=0), dict(K=17), dict(H=1000), dict(H=9216),
           dict(H=1024 + 16), dict(eps=-1.0), dict(eps=float("inf")), dict(eps=float("nan")),
           dict(mode=2), dict(eo=None), dict(asg=None), dict(s=None), dict(res=None),
           dict(g=None), dict(y=None), dict(eo=P + 8), dict(y=P + 2), dict(sh=P + 8),
           dict(xo=P + 8), dict(asg=P + 2), dict(rstd=P + 1)]
    for kw in bad:
        assert combine(**kw) == 1, kw


@pytest.mark.skipif("not _no_gpu()")
def test_update_expert_rejects_out_of_range_arguments():
    u = limits()["update_expert_shapes"]
    bad = [dict(Bs=0), dict(Bs=u["Bs"]["max"] + 1), dict(K=0), dict(K=17),
           dict(nl=0), dict(nl=u["moeExpertNum"]["max"] + 1), dict(nl=8, K=16),
           dict(F=1), dict(F=514), dict(ni=0), dict(ni=u["total_instances_max"] + 1),
           dict(ids=None), dict(t=None), dict(oi=None), dict(om=None), dict(ids=P + 2),
           dict(sc=P + 1), dict(thr=P + 3)]
    for kw in bad:
        assert update(**kw) == 1, kw


def fused(**kw):
    from combine_expert_amd import moe
    a = dict(x=P, ids=P, sc=None, t=P, thr=None, tm=None, Bs=512, H=8192, K=16, nl=512, F=3,
             R=64, L=16, q=3, tile=128, qs=None, qk=0, bi=None, bm=None, ex=P, esc=P, cnt=P,
             off=P, src=P, asg=P, err=None)
    a.update(kw)
    return moe.raw().moe_update_dispatch(a["x"], a["ids"], a["sc"], a["t"], a["thr"], a["tm"],
                                         a["Bs"], a["H"], a["K"], a["nl"], a["F"], a["R"],
                                         a["L"], a["q"], a["tile"], a["qs"], a["qk"], a["bi"],
                                         a["bm"], a["ex"], a["esc"], a["cnt"], a["off"],
                                         a["src"], a["asg"], a["err"], None)


@pytest.mark.skipif("not _no_gpu()")
def test_fused_update_dispatch_rejects_out_of_range_arguments():
    bad = [dict(Bs=0), dict(K=17), dict(H=7168 + 16), dict(t=None), dict(nl=0), dict(nl=1025),
           dict(nl=8, K=16), dict(F=1), dict(F=514), dict(R=0), dict(R=65), dict(x=None),
           dict(ids=None), dict(ids=P + 4), dict(sc=P + 4, thr=P), dict(thr=P + 1),
           dict(bi=P + 2), dict(q=3, tile=0), dict(q=7), dict(asg=None), dict(q=1),
           dict(q=3, qs=P, qk=1), dict(q=5, esc=None)]
    for kw in bad:
        assert fused(**kw) == 1, kw
    # a table too large to stage in LDS, odd tiles: not supported
    for kw in (dict(nl=1024, F=13, K=16), dict(q=3, tile=96)):
        assert fused(**kw) == 2, kw


def gemm(**kw):
    from combine_expert_amd import moe
    a = dict(a=P, asc=P, off=P, E=8, rows=4096, w=P, wsc=P, N=4096, H=7168, q=4, y=P, err=None)
    a.update(kw)
    return moe.raw().moe_expert_gemm(a["a"], a["asc"], a["off"], a["E"], a["rows"], a["w"],
                                     a["wsc"], a["N"], a["H"], a["q"], a["y"], a["err"], None)


@pytest.mark.skipif("not _no_gpu()")
def test_expert_gemm_rejects_out_of_range_arguments():
    bad = [dict(a=None), dict(asc=None), dict(off=None), dict(w=None), dict(wsc=None),
           dict(y=None), dict(E=0), dict(E=1025), dict(rows=-1), dict(rows=(1 << 22) + 1),
           dict(H=7168 + 32), dict(H=0),
           dict(H=16384 + 128), dict(N=100), dict(N=0), dict(N=16384 + 128), dict(q=7),
           dict(q=-1), dict(a=P + 8), dict(w=P + 4), dict(y=P + 8), dict(asc=P + 2),
           dict(wsc=P + 1), dict(off=P + 2), dict(err=P + 1)]
    for kw in bad:
        assert gemm(**kw) == 1, kw
    for q in (0, 1, 6):
        assert gemm(q=q) == 2, q


def swiglu(**kw):
    from combine_expert_amd import moe
    a = dict(y1=P, off=P, E=8, rows=4096, I=2048, q=4, codes=P, sc=P, act=None, err=None)
    a.update(kw)
    return moe.raw().moe_expert_swiglu(a["y1"], a["off"], a["E"], a["rows"], a["I"], a["q"],
                                       a["codes"], a["sc"], a["act"], a["err"], None)


@pytest.mark.skipif("not _no_gpu()")
def test_expert_swiglu_rejects_out_of_range_arguments():
    bad = [dict(y1=None), dict(off=None), dict(codes=None), dict(sc=None), dict(E=0),
           dict(E=1025), dict(rows=-1), dict(rows=(1 << 22) + 1), dict(I=0), dict(I=64),
           dict(I=2000), dict(I=8192 + 128), dict(q=-1), dict(q=7), dict(y1=P + 8),
           dict(codes=P + 4), dict(act=P + 8), dict(off=P + 2), dict(err=P + 1)]
    for kw in bad:
        assert swiglu(**kw) == 1, kw
    for q in (0, 1, 2, 3, 6):
        assert swiglu(q=q) == 2, q
    # valid calls reach the launch (no GPU here: the launch itself fails)
    for kw in (dict(), dict(q=5), dict(I=128), dict(I=8192), dict(act=P)):
        assert swiglu(**kw) == 3, kw
    assert swiglu(rows=0) == 0  # nothing to launch
