"""Helpers for the GPU parity tests: run a stage through the C ABI and run the
same stage through the CPU oracle on the same seeded inputs.

Tolerances (floating-point outputs of the combine): |gpu - oracle| <=
2e-2 + 1e-2 * |oracle| elementwise for the bf16 outputs y and x_out (fp32
accumulation on the GPU, fp64 in the oracle), 1e-4 relative for rstd.
Everything integer (ids, masks, counts, offsets, rows, codes, scales) must be
bit-exact.
"""
import sys

import numpy as np
import torch

import oracle
from combine_expert_amd import workloads as W

ABS_TOL = 2e-2
REL_TOL = 1e-2
RSTD_RTOL = 1e-4
POISON = 0xAB


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def M():
    from combine_expert_amd import moe
    return moe


def cuda(t):
    return None if t is None else t.contiguous().cuda()


def np_(t):
    return None if t is None else t.detach().cpu().numpy()


def bits(t):
    return oracle.bf16_bits(t)


def f32_of_bits(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32)


def gpu_update(wl, dev_err=None):
    m = M()
    ids, mask = m.moe_update_expert(cuda(wl.logical_ids), cuda(wl.table), wl.E,
                                    expert_scales=cuda(wl.scales) if wl.prune_thr is not None
                                    else None,
                                    prune_thr=cuda(wl.prune_thr), token_mask=cuda(wl.token_mask),
                                    dev_err=dev_err)
    return ids, mask


def oracle_update(wl):
    return oracle.update_expert(wl.logical_ids.numpy(),
                                wl.scales.numpy() if wl.prune_thr is not None else None,
                                wl.table.numpy(),
                                None if wl.prune_thr is None else wl.prune_thr.numpy(),
                                None if wl.token_mask is None else wl.token_mask.numpy(), wl.E)


def gpu_dispatch(wl, ids, mask, x=None, poison=True, dev_err=None):
    m = M()
    x = cuda(wl.x) if x is None else x
    out = m.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile)
    if poison:
        for key in ("expand_x", "expand_scales"):
            if out.get(key) is not None:
                out[key].view(torch.uint8).fill_(POISON)
        for key in ("expert_counts", "expert_offsets", "expand_src", "assist_dst"):
            out[key].fill_(-7)
    return m.moe_dispatch(x, ids, wl.n_ranks, wl.local_experts, wl.quant_mode, wl.tile,
                          active_mask=mask, out=out, dev_err=dev_err)


QUANT_MXFP8_GM = 5  # the mxfp8 codes with the exponents stored group-major


def oracle_dispatch(wl, ids, mask, x_bits=None):
    """The oracle's dispatch; the group-major mxfp8 mode is the mxfp8 case of the pages
    stored in another order, so the oracle computes case 5 and check_dispatch permutes."""
    xb = bits(wl.x) if x_bits is None else x_bits
    mode = 4 if wl.quant_mode == QUANT_MXFP8_GM else wl.quant_mode
    return oracle.dispatch(xb, ids, mask, wl.n_ranks, wl.local_experts, mode, wl.tile)


def gm_to_row_major(gm, N, H):
    """Group-major exponents [ceil(H/512), N, 16] -> row-major [N, H/32] (a permutation;
    the pad bytes of a partial last group are dropped)."""
    G = -(-H // 512)
    g = np.asarray(gm, dtype=np.uint8).reshape(G, N, 16)
    return np.ascontiguousarray(g.transpose(1, 0, 2).reshape(N, G * 16)[:, :H // 32])


def row_major_to_gm(sc, H):
    """Row-major exponents [N, H/32] -> group-major [ceil(H/512), N, 16]; the pad bytes of a
    partial last group hold 0xFF (the E8M0 NaN), which no reader may use."""
    sc = np.asarray(sc, dtype=np.uint8)
    N = sc.shape[0]
    G = -(-H // 512)
    padded = np.full((N, G * 16), 0xFF, np.uint8)  # pad: E8M0 NaN, never read
    padded[:, :H // 32] = sc
    return np.ascontiguousarray(padded.reshape(N, G, 16).transpose(1, 0, 2))


def check_dispatch(wl, g, o):
    """Bit-exact comparison of a GPU dispatch against the oracle's."""
    N = wl.Bs * wl.K
    np.testing.assert_array_equal(np_(g["expert_counts"]), o["counts"])
    np.testing.assert_array_equal(np_(g["expert_offsets"]), o["offsets"])
    np.testing.assert_array_equal(np_(g["assist_dst"]), o["assist"])
    np.testing.assert_array_equal(np_(g["expand_src"]), o["src"])
    total = int(o["offsets"][-1])
    gx = g["expand_x"].view(torch.uint8).cpu().numpy().reshape(N, -1)
    ox = o["expand_x"].view(np.uint8).reshape(N, -1)
    np.testing.assert_array_equal(gx[:total], ox[:total])
    assert np.all(gx[total:] == POISON), "rows past the total were written"
    if o["scales"] is not None:
        os_ = o["scales"].view(np.uint8).reshape(N, -1)
        if wl.quant_mode == QUANT_MXFP8_GM:
            G = -(-wl.H // 512)
            raw = g["expand_scales"].view(torch.uint8).cpu().numpy().reshape(G, N, 16)
            gs = gm_to_row_major(raw, N, wl.H)
            pad = raw.transpose(1, 0, 2).reshape(N, G * 16)[:, wl.H // 32:]
            assert np.all(pad == POISON), "pad bytes of the last group were written"
        else:
            gs = g["expand_scales"].view(torch.uint8).cpu().numpy().reshape(N, -1)
        np.testing.assert_array_equal(gs[:total], os_[:total])
        assert np.all(gs[total:] == POISON)
    return total


def gpu_combine(wl, assist, eout, residual=None, shared_mode=None):
    m = M()
    res = wl.residual if residual is None else residual
    y, xo, rstd = m.moe_combine_add_rmsnorm(
        cuda(eout), cuda(assist).reshape(wl.Bs, wl.K), cuda(wl.scales), cuda(res),
        cuda(wl.gamma), wl.eps, shared_x=cuda(wl.shared),
        shared_mode=wl.shared_mode if shared_mode is None else shared_mode)
    return y, xo, rstd


def oracle_combine(wl, assist, eout, residual=None, shared_mode=None):
    res = wl.residual if residual is None else residual
    return oracle.combine(bits(eout), np.asarray(assist).reshape(wl.Bs, wl.K), wl.scales.numpy(),
                          None if wl.shared is None else bits(wl.shared), bits(res),
                          bits(wl.gamma), wl.eps,
                          wl.shared_mode if shared_mode is None else shared_mode)


def check_close_bf16(gpu_t, oracle_bits, what):
    g = gpu_t.float().cpu().numpy()
    o = f32_of_bits(oracle_bits).astype(np.float64)
    err = np.abs(g - o)
    lim = ABS_TOL + REL_TOL * np.abs(o)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3e}")
    return float(err.max())


def check_combine(g, o):
    y, xo, rstd = g
    oy, oxo, orstd = o
    check_close_bf16(y, oy, "y")
    check_close_bf16(xo, oxo, "x_out")
    np.testing.assert_allclose(rstd.cpu().numpy(), orstd, rtol=RSTD_RTOL)
