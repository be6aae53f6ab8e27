"""One MoE layer as a chain on the GPU: the mapping, the mxfp8 dispatch, the
expert computation as one linear layer of width H per instance
(moe_expert_gemm with N = H, so that its output is the expert_out the combine
reads, rows in dispatch order), then the combine with shared expert,
residual and RMSNorm.  Each stage is checked against the oracle on the GPU's
own inputs to that stage: mapping and dispatch bit for bit, the expert GEMM
within its tolerance and mostly bit-equal to the oracle's bf16, the combine
within its tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import (M, check_combine, check_dispatch, gpu_combine, gpu_dispatch,
                              gpu_update, np_, oracle_combine, oracle_dispatch, oracle_update,
                              say)
from tests.test_gpu_gemm import BIT_EQUAL_MIN, assert_close

pytestmark = pytest.mark.gpu

CASES = [
    # seed, Bs, H, K, ranks, local experts
    (801, 37, 1024, 4, 2, 4),
    (802, 256, 2048, 8, 8, 8),
]


def expert_weights(seed, E, H):
    """Synthetic mxfp8 weights [E, H, H] (E4M3 codes, E8M0 exponents per 32 along K)."""
    rng = np.random.default_rng(seed)
    return W.e4m3_codes(rng, (E, H, H)), W.e8m0_codes(rng, (E, H, H // 32), 110, 114)


@pytest.mark.parametrize("case", CASES, ids=[f"chain{c[0]}" for c in CASES])
def test_layer_chain(case):
    seed, Bs, H, K, R, L = case
    m = M()
    wl = W.make_small(seed, Bs, H, K, R, L, W.QUANT_MXFP8)
    E = wl.E
    say(f"[chain] {case}: mapping and dispatch")
    gi, gm = gpu_update(wl)
    oi, om, _ = oracle_update(wl)
    np.testing.assert_array_equal(np_(gi), oi)
    np.testing.assert_array_equal(np_(gm), om)
    gd = gpu_dispatch(wl, gi, gm)
    od = oracle_dispatch(wl, oi, om)
    total = check_dispatch(wl, gd, od)

    say(f"[chain] {case}: expert GEMM, {total} rows x {H} x {H}")
    w, w_sc = expert_weights(seed + 1, E, H)
    y = torch.full((Bs * K, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(gd["expand_x"], gd["expand_scales"], gd["expert_offsets"],
                      torch.from_numpy(w).cuda(),
                      m.pack_mx_weight_scales(torch.from_numpy(w_sc).cuda()), y=y)
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    a = od["expand_x"].view(np.uint8)[:total]
    a_sc = od["scales"].view(np.uint8)[:total]
    offsets = od["offsets"]
    rows = np.arange(total) if total <= 512 else np.unique(np.concatenate([
        offsets[:-1][np.diff(offsets) > 0], offsets[1:][np.diff(offsets) > 0] - 1,
        np.random.default_rng(seed + 2).integers(0, total, 128)]))
    inst = np.searchsorted(offsets, rows, side="right") - 1
    sub_off = np.zeros(E + 1, np.int32)
    sub_off[1:] = np.cumsum(np.bincount(inst, minlength=E))
    ref, y64, abs64 = oracle.expert_gemm_mx(a[rows], a_sc[rows], sub_off, w, w_sc)
    assert_close(yb[rows], y64, abs64, H, f"chain {seed} GEMM")
    assert np.mean(yb[rows] == ref) > BIT_EQUAL_MIN

    say(f"[chain] {case}: combine on the GEMM's output")
    g = gpu_combine(wl, gd["assist_dst"], y.cpu())
    o = oracle_combine(wl, od["assist"], y.cpu())
    check_combine(g, o)
