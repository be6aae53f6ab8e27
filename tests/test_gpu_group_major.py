"""GPU parity of the group-major mxfp8 layout (quant mode 5): the dispatch writes
the mxfp8 codes and exponents of case 5 of the dispatch page with the
exponents stored [ceil(H/512)][rows][16], and the expert GEMM reads them there.

The oracle computes case 5 (row-major exponents); the tests permute on the host:
  - dispatch, separate and fused calls: every output bit for bit against the
    oracle, the exponents after the permutation, and the pad bytes of a partial
    last group and the rows past the total untouched;
  - GEMM: the same bar as the row-major GEMM tests against the oracle, and the
    output bit for bit equal to the row-major launch on the same operands (only
    the addresses of the exponent copies differ), with the pad bytes set to the
    E8M0 NaN so that a read of one shows;
  - the chain dispatch -> GEMM on the dispatch's own output.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import (M, QUANT_MXFP8_GM, cuda, gpu_update, np_, oracle_dispatch,
                              oracle_update, row_major_to_gm, say)
from tests.test_gpu_fused import check_fused
from tests.test_gpu_gemm import (BIT_EQUAL_MIN, POISON16, assert_close, check_sampled)
from tests.test_gpu_parity import full_chain

pytestmark = pytest.mark.gpu

DISPATCH_CASES = [
    # seed, Bs, H, K, ranks, local, prune, token-mask prefix, replicas
    (901, 37, 1056, 5, 3, 4, True, None, False),     # 33 blocks: last group holds one
    (902, 19, 2080, 3, 2, 3, False, None, False),    # 65 blocks: last group holds one
    (903, 64, 1536, 7, 5, 5, True, 40, True),        # three whole groups
    (904, 512, 7168, 8, 32, 8, True, 400, True),     # the headline shape
    (905, 512, 8192, 16, 64, 16, True, None, True),  # 8192 entries: two launches fused
    (906, 1, 8192, 16, 128, 8, False, None, False),
]


@pytest.mark.parametrize("case", DISPATCH_CASES, ids=[f"gm{c[0]}" for c in DISPATCH_CASES])
def test_dispatch_group_major(case):
    seed, Bs, H, K, R, L, prune, prefix, rep = case
    wl = W.make_small(seed, Bs, H, K, R, L, QUANT_MXFP8_GM, prune=prune,
                      token_mask_prefix=prefix, replicas=rep)
    say(f"[group-major] dispatch {case}: separate calls")
    full_chain(wl)
    say(f"[group-major] dispatch {case}: fused call")
    check_fused(wl)


def test_dispatch_group_major_equals_row_major_permuted():
    """The same call in modes 4 and 5: codes and routing bit for bit equal, exponents a
    permutation of each other (headline shape)."""
    m = M()
    wl = W.make_c3(quant_mode=4)
    say("[group-major] modes 4 and 5 on c3")
    outs = {}
    for mode in (4, QUANT_MXFP8_GM):
        outs[mode] = m.moe_update_dispatch(
            cuda(wl.x), cuda(wl.logical_ids), cuda(wl.table), wl.n_ranks, wl.local_experts,
            mode, 0, expert_scales=cuda(wl.scales) if wl.prune_thr is not None else None,
            prune_thr=cuda(wl.prune_thr) if wl.prune_thr is not None else None,
            token_mask=cuda(wl.token_mask))
    torch.cuda.synchronize()
    a, b = outs[4], outs[QUANT_MXFP8_GM]
    total = int(a["expert_offsets"][-1].item())
    for key in ("expert_counts", "expert_offsets", "expand_src", "assist_dst",
                "balanced_ids", "balanced_mask"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["expand_x"][:total], b["expand_x"][:total])
    N, G = wl.Bs * wl.K, -(-wl.H // 512)
    ra = np_(a["expand_scales"]).reshape(N, wl.H // 32)[:total]
    rb = row_major_view(np_(b["expand_scales"]), N, wl.H)[:total]
    np.testing.assert_array_equal(ra, rb)
    assert b["expand_scales"].shape == (G, N, 16)


def row_major_view(gm, N, H):
    G = -(-H // 512)
    return gm.reshape(G, N, 16).transpose(1, 0, 2).reshape(N, G * 16)[:, :H // 32]


# ------------------------------------------------------------------------- GEMM

def run_gemm(g, quant_mode):
    m = M()
    sc = g.a_sc if quant_mode == 4 else row_major_to_gm(g.a_sc, g.Kd)
    y = torch.full((g.rows, g.N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    m.moe_expert_gemm(torch.from_numpy(g.a).cuda(), torch.from_numpy(sc).cuda(),
                      torch.from_numpy(np.ascontiguousarray(g.offsets, np.int32)).cuda(),
                      torch.from_numpy(g.w).cuda(),
                      m.pack_mx_weight_scales(torch.from_numpy(g.w_sc).cuda()), quant_mode, y=y)
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


GEMM_CASES = [
    # (seed, counts per instance, N, Kd, tail rows): Kd not a multiple of 512 takes the
    # per-step exponent copies (the pad bytes of the last group are then next to what
    # is read), multiples of 512 the grouped copies
    (950, [0, 17, 130, 1, 255], 256, 256, 5),
    (951, [1, 129, 64], 384, 384, 0),
    (952, [3, 0, 0, 7, 0, 200, 0, 1], 128, 512, 2),
    (953, [5, 260, 0, 131], 256, 1536, 1),
    (954, [300, 41], 256, 1152, 3),
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[f"g{c[0]}" for c in GEMM_CASES])
def test_gemm_group_major_small(case):
    seed, counts, N, Kd, tail = case
    say(f"[group-major] GEMM {case}")
    g = W.make_gemm_case(seed, counts, N, Kd, tail=tail)
    y = run_gemm(g, QUANT_MXFP8_GM)
    ref, y64, abs64 = oracle.expert_gemm_mx(g.a, g.a_sc, g.offsets, g.w, g.w_sc)
    last = int(g.offsets[-1])
    assert_close(y[:last], y64[:last], abs64[:last], Kd, f"group-major {seed}")
    assert np.all(y[last:] == POISON16)
    if last:
        assert np.mean(y[:last] == ref[:last]) > BIT_EQUAL_MIN
    np.testing.assert_array_equal(y, run_gemm(g, 4))


def test_gemm_group_major_full_size_and_wide():
    """The bench shape (narrow tiling) and a shape the 256 x 256 tiling takes: sampled
    against the oracle and bit for bit equal to the row-major launch."""
    for g, where in ((W.make_g3(), "bench shape"),
                     (W.make_gemm_case(7212, [3000, 1500, 2600, 700], 2048, 512, tail=17),
                      "wide tiling")):
        say(f"[group-major] GEMM {where}: counts={g.counts.tolist()} N={g.N} Kd={g.Kd}")
        y = run_gemm(g, QUANT_MXFP8_GM)
        check_sampled(g, y, where=f"group-major {where}")
        np.testing.assert_array_equal(y, run_gemm(g, 4))


def test_chain_dispatch_to_gemm_group_major():
    """The dispatch's group-major output fed straight to the GEMM: equal bit for bit to
    the row-major chain on the same routing, and within tolerance of the oracle."""
    m = M()
    Bs, H, K, R, L = 256, 2048, 8, 8, 8
    wl = W.make_small(811, Bs, H, K, R, L, 4, prune=True)
    rng = np.random.default_rng(812)
    E = wl.E
    w = W.e4m3_codes(rng, (E, H, H))
    w_sc = W.e8m0_codes(rng, (E, H, H // 32), 110, 114)
    wt, wsc = torch.from_numpy(w).cuda(), m.pack_mx_weight_scales(torch.from_numpy(w_sc).cuda())
    gi, gmask = gpu_update(wl)
    ys = {}
    for mode in (4, QUANT_MXFP8_GM):
        say(f"[group-major] chain, mode {mode}")
        d = m.moe_dispatch(cuda(wl.x), gi, wl.n_ranks, wl.local_experts, mode, 0,
                           active_mask=gmask)
        y = torch.full((Bs * K, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        m.moe_expert_gemm(d["expand_x"], d["expand_scales"], d["expert_offsets"], wt, wsc,
                          mode, y=y)
        torch.cuda.synchronize()
        ys[mode] = y.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(ys[4], ys[QUANT_MXFP8_GM])
    oi, om, _ = oracle_update(wl)
    od = oracle_dispatch(wl, oi, om)
    total = int(od["offsets"][-1])
    assert total > 0
    rows = np.unique(np.random.default_rng(813).integers(0, total, 96))
    offsets = od["offsets"]
    inst = np.searchsorted(offsets, rows, side="right") - 1
    sub_off = np.zeros(E + 1, np.int32)
    sub_off[1:] = np.cumsum(np.bincount(inst, minlength=E))
    a = od["expand_x"].view(np.uint8)[:total]
    a_sc = od["scales"].view(np.uint8)[:total]
    ref, y64, abs64 = oracle.expert_gemm_mx(a[rows], a_sc[rows], sub_off, w, w_sc)
    yb = ys[QUANT_MXFP8_GM]
    assert_close(yb[rows], y64, abs64, H, "group-major chain")
    assert np.mean(yb[rows] == ref) > BIT_EQUAL_MIN


def test_gemm_group_major_limits():
    """The group pitch at the limits: K = 16384 (32 groups of exponents, the last group at
    31 pitches), and 4194304 rows (a 64 MB group pitch; H = 128 reads part of one group,
    so the per-step copies run), sampled against the oracle and equal to the row-major
    launch on the sampled rows."""
    g = W.make_gemm_case(7103, [200, 77, 129], 256, 16384)
    say("[group-major] GEMM K = 16384")
    y = run_gemm(g, QUANT_MXFP8_GM)
    check_sampled(g, y, where="group-major K=16384")
    np.testing.assert_array_equal(y, run_gemm(g, 4))
    g = W.make_gemm_case(7106, [4194304 - 1000, 1000], 128, 128)
    say("[group-major] GEMM 4194304 rows")
    y = run_gemm(g, QUANT_MXFP8_GM)
    extra = np.random.default_rng(7107).integers(0, g.rows, 64)
    check_sampled(g, y, extra_rows=extra, where="group-major 4M rows")
    rows = np.unique(np.concatenate([extra, [0, g.rows - 1]]))
    np.testing.assert_array_equal(y[rows], run_gemm(g, 4)[rows])
