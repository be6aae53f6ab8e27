"""GPU parity of the expert FFN's activation (moe_expert_swiglu) and of one
layer with the whole FFN: mapping, mxfp8 dispatch, the first projection
(moe_expert_gemm, N = 2I: gate | up), the activation with its mxfp8 coding,
the second projection (N = H: the combine's expert_out) and the combine.

The activation is bf16(silu(gate) * up) in fp32 on the GPU and in fp64 in the
oracle, so a value near a bf16 rounding midpoint may round one step apart:
the test allows that on at most 1e-3 of the elements, one step and the same
sign each.  The codes and exponents must then equal, bit for bit, the case-5
quantiser of the oracle applied to the GPU's own bf16 act.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import (M, POISON, QUANT_MXFP8_GM, check_combine, check_dispatch,
                              gm_to_row_major, gpu_combine, gpu_dispatch, gpu_update, np_,
                              oracle_combine, oracle_dispatch, oracle_update, say)
from tests.test_gpu_gemm import BIT_EQUAL_MIN, assert_close

pytestmark = pytest.mark.gpu

ACT_MISMATCH_MAX = 1e-3


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_act(act_gpu, act_ref, where):
    """bf16 patterns: equal, or adjacent with the same sign on a small fraction."""
    a = act_gpu.astype(np.int32)
    b = act_ref.astype(np.int32)
    diff = a != b
    frac = diff.mean() if diff.size else 0.0
    say(f"{where}: {diff.sum()} of {diff.size} act values one bf16 step from the oracle's")
    assert frac <= ACT_MISMATCH_MAX, f"{where}: {diff.sum()} of {diff.size} act values differ"
    if diff.any():
        same_sign = (a[diff] & 0x8000) == (b[diff] & 0x8000)
        assert same_sign.all() and (np.abs(a[diff] - b[diff]) == 1).all(), \
            f"{where}: act differs by more than one bf16 step"


def codes_of(act_bits):
    """The oracle's case-5 quantiser on bf16 rows: each row is one token of a dispatch
    with one instance and K = 1 (the rows come out in order)."""
    rows, I = act_bits.shape
    o = oracle.dispatch(act_bits, np.zeros((rows, 1), np.int32), None, 1, 1, 4)
    return o["expand_x"].view(np.uint8), o["scales"]


def run_swiglu(y1, offsets, mode, rows, I):
    m = M()
    codes = torch.full((rows, I), POISON, dtype=torch.uint8, device="cuda")
    ns = m.n_scale_entries(mode, I)
    shape = (ns // 16, rows, 16) if mode == QUANT_MXFP8_GM else (rows, ns)
    sc = torch.full(shape, POISON, dtype=torch.uint8, device="cuda")
    act = torch.full((rows, I), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.moe_expert_swiglu(y1, offsets, mode, act_codes=codes, act_scales=sc, act=act, dev_err=err)
    torch.cuda.synchronize()
    sc_np = sc.cpu().numpy()
    if mode == QUANT_MXFP8_GM:
        G = -(-I // 512)
        pad = sc_np.reshape(G, rows, 16).transpose(1, 0, 2).reshape(rows, G * 16)[:, I // 32:]
        assert (pad == POISON).all(), "pad bytes of the last exponent group were written"
        sc_np = gm_to_row_major(sc_np, rows, I)
    return codes.cpu().numpy(), sc_np, u16(act), int(err.item())


CASES = [
    # seed, row capacity, offsets, I, mode (4 row-major exponents, 5 group-major)
    (901, 97, [0, 20, 20, 60], 128, 4),
    (902, 300, [0, 100, 260], 640, 5),      # a partial last exponent group (20 blocks)
    (903, 512, [0, 512], 2048, 5),
    (904, 64, [0, 7, 33, 64], 8192, 4),
]


@pytest.mark.parametrize("case", CASES, ids=[f"swiglu{c[0]}" for c in CASES])
def test_swiglu_against_oracle(case):
    seed, rows, off, I, mode = case
    say(f"[ffn] swiglu {case}")
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, 3.0, size=(rows, I))
    g[::5, ::7] *= 40.0                      # large gates: silu(g) = g, or an underflow to -0
    u = rng.normal(0.0, 2.0, size=(rows, I))
    y1 = torch.from_numpy(np.concatenate([g, u], axis=1).astype(np.float32)).bfloat16()
    offsets = np.array(off, np.int32)
    codes, sc, act, err = run_swiglu(y1.cuda(), torch.from_numpy(offsets).cuda(), mode, rows, I)
    assert err == 0
    lo, hi = off[0], off[-1]
    ref_act, _, _ = oracle.swiglu_mx(oracle.bf16_bits(y1), offsets)
    check_act(act[lo:hi], ref_act[lo:hi], f"swiglu {seed}")
    rc, rs = codes_of(act[lo:hi])
    np.testing.assert_array_equal(codes[lo:hi], rc)
    np.testing.assert_array_equal(sc[lo:hi], rs)
    for t, v in ((codes, POISON), (sc, POISON), (act, 0xFFFF)):
        assert (t[:lo] == v).all() and (t[hi:] == v).all(), "rows outside the range were written"


def test_swiglu_rejects_bad_offsets_without_leaving_the_buffers():
    say("[ffn] swiglu, offsets past the rows")
    rows, I = 40, 256
    y1 = torch.randn(rows, 2 * I).bfloat16().cuda()
    codes, sc, act, err = run_swiglu(y1, torch.tensor([0, 50], dtype=torch.int32).cuda(), 4,
                                     rows, I)
    assert err == 16  # MOE_ERR_OFFSETS; rows clamped to [0, 40)
    rc, rs = codes_of(act)
    np.testing.assert_array_equal(codes, rc)


def mx_weights(seed, E, N, K):
    rng = np.random.default_rng(seed)
    return W.e4m3_codes(rng, (E, N, K)), W.e8m0_codes(rng, (E, N, K // 32), 110, 114)


def check_gemm_rows(y_bits, a, a_sc, offsets, w, w_sc, Kd, seed, where):
    """Sampled rows of a GEMM output against the oracle on the same operands."""
    E = offsets.size - 1
    total = int(offsets[-1])
    rows = np.arange(total) if total <= 256 else np.unique(np.concatenate([
        offsets[:-1][np.diff(offsets) > 0], offsets[1:][np.diff(offsets) > 0] - 1,
        np.random.default_rng(seed).integers(0, total, 96)]))
    inst = np.searchsorted(offsets, rows, side="right") - 1
    sub = np.zeros(E + 1, np.int32)
    sub[1:] = np.cumsum(np.bincount(inst, minlength=E))
    ref, y64, abs64 = oracle.expert_gemm_mx(a[rows], a_sc[rows], sub, w, w_sc)
    assert_close(y_bits[rows], y64, abs64, Kd, where)
    assert np.mean(y_bits[rows] == ref) > BIT_EQUAL_MIN


FFN_CASES = [
    # seed, Bs, H, K, ranks, local experts, I
    (911, 37, 1024, 4, 2, 4, 256),
    (912, 128, 2048, 8, 4, 8, 512),
]


@pytest.mark.parametrize("case", FFN_CASES, ids=[f"ffn{c[0]}" for c in FFN_CASES])
def test_layer_with_the_ffn(case):
    seed, Bs, H, K, R, L, I = case
    m = M()
    wl = W.make_small(seed, Bs, H, K, R, L, W.QUANT_MXFP8)
    E, N = wl.E, Bs * K
    say(f"[ffn] {case}: mapping and dispatch")
    gi, gm = gpu_update(wl)
    oi, om, _ = oracle_update(wl)
    np.testing.assert_array_equal(np_(gi), oi)
    gd = gpu_dispatch(wl, gi, gm)
    od = oracle_dispatch(wl, oi, om)
    total = check_dispatch(wl, gd, od)
    offsets = od["offsets"]

    say(f"[ffn] {case}: first projection, {total} rows x {2 * I} x {H}")
    w1, w1_sc = mx_weights(seed + 1, E, 2 * I, H)
    y1 = torch.full((N, 2 * I), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(gd["expand_x"], gd["expand_scales"], gd["expert_offsets"],
                      torch.from_numpy(w1).cuda(),
                      m.pack_mx_weight_scales(torch.from_numpy(w1_sc).cuda()), y=y1)
    y1b = u16(y1)
    a, a_sc = od["expand_x"].view(np.uint8)[:total], od["scales"].view(np.uint8)[:total]
    check_gemm_rows(y1b, a, a_sc, offsets, w1, w1_sc, H, seed + 2, f"ffn {seed} first")

    say(f"[ffn] {case}: activation, group-major exponents for the second projection")
    codes, sc, act, err = run_swiglu(y1, gd["expert_offsets"], QUANT_MXFP8_GM, N, I)
    assert err == 0
    ref_act, _, _ = oracle.swiglu_mx(y1b, offsets)
    check_act(act[:total], ref_act[:total], f"ffn {seed} act")
    rc, rs = codes_of(act[:total])
    np.testing.assert_array_equal(codes[:total], rc)
    np.testing.assert_array_equal(sc[:total], rs)

    say(f"[ffn] {case}: second projection, {total} rows x {H} x {I}")
    w2, w2_sc = mx_weights(seed + 3, E, H, I)
    codes_d, sc_d, _ = m.moe_expert_swiglu(y1, gd["expert_offsets"], QUANT_MXFP8_GM)
    y2 = torch.full((N, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(codes_d, sc_d, gd["expert_offsets"], torch.from_numpy(w2).cuda(),
                      m.pack_mx_weight_scales(torch.from_numpy(w2_sc).cuda()),
                      quant_mode=QUANT_MXFP8_GM, y=y2)
    y2b = u16(y2)
    check_gemm_rows(y2b, codes[:total], sc[:total], offsets, w2, w2_sc, I, seed + 4,
                    f"ffn {seed} second")

    say(f"[ffn] {case}: combine on the FFN's output")
    g = gpu_combine(wl, gd["assist_dst"], y2.cpu())
    o = oracle_combine(wl, od["assist"], y2.cpu())
    check_combine(g, o)


def test_swiglu_is_bitwise_repeatable():
    say("[ffn] swiglu twice on the same input")
    rows, I = 256, 1024
    rng = np.random.default_rng(905)
    y1 = torch.from_numpy(rng.normal(0.0, 4.0, size=(rows, 2 * I)).astype(np.float32))
    y1 = y1.bfloat16().cuda()
    off = torch.tensor([0, 100, 256], dtype=torch.int32).cuda()
    a = run_swiglu(y1, off, QUANT_MXFP8_GM, rows, I)
    b = run_swiglu(y1, off, QUANT_MXFP8_GM, rows, I)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


def test_ffn_replays_from_a_graph():
    """The rank's FFN (first projection, activation, second projection) captured in one
    HIP graph: every replay, with eager work between them, equals the eager run bitwise."""
    say("[ffn] graph capture and replays")
    m = M()
    rng = np.random.default_rng(906)
    E, H, I = 4, 1024, 256
    counts = np.array([40, 0, 130, 86], np.int32)
    rows = int(counts.sum()) + 8
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    a = torch.from_numpy(W.e4m3_codes(rng, (rows, H))).cuda()
    a_sc = torch.from_numpy(W.e8m0_codes(rng, (rows, H // 32), 120, 124)).cuda()
    w1, w1_sc = mx_weights(907, E, 2 * I, H)
    w2, w2_sc = mx_weights(908, E, H, I)
    w1, w2 = torch.from_numpy(w1).cuda(), torch.from_numpy(w2).cuda()
    w1_sc = m.pack_mx_weight_scales(torch.from_numpy(w1_sc).cuda())
    w2_sc = m.pack_mx_weight_scales(torch.from_numpy(w2_sc).cuda())
    y1 = torch.zeros((rows, 2 * I), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((rows, I), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((-(-I // 512), rows, 16), dtype=torch.uint8, device="cuda")
    y2 = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")

    def ffn():
        m.moe_expert_gemm(a, a_sc, off, w1, w1_sc, y=y1)
        m.moe_expert_swiglu(y1, off, QUANT_MXFP8_GM, act_codes=codes, act_scales=sc)
        m.moe_expert_gemm(codes, sc, off, w2, w2_sc, quant_mode=QUANT_MXFP8_GM, y=y2)

    total = int(counts.sum())  # the spare rows past it are written by no kernel
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ffn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (u16(y1)[:total], codes.cpu().numpy()[:total], sc.cpu().numpy(), u16(y2)[:total])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ffn()
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for t in (y1, y2):
            t.view(torch.int16).fill_(rep + 1)
        codes.fill_(rep + 7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (u16(y1)[:total], codes.cpu().numpy()[:total], sc.cpu().numpy(), u16(y2)[:total])
        for x, y in zip(ref, got):
            np.testing.assert_array_equal(x, y)
        other.mul_(1.0001).add_(0.5)
        ffn()
        torch.cuda.synchronize()
