"""GPU parity of moe_update_dispatch, the expert mapping fused into the
dispatch launch: its balanced ids / mask and every dispatch output against
the oracle's update_expert followed by its dispatch (bit for bit), and
against the two separate GPU calls, with the same device error bits.

Cases: the five workloads at full size, small ragged shapes with pruning,
prefix token masks, replica tables and every quantisation mode, a table at
the staging limit, and malformed input (out-of-range ids, bad table rows,
an illegal 1-D token mask).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import (M, POISON, check_dispatch, cuda, gpu_dispatch, gpu_update, np_,
                              oracle_dispatch, oracle_update, say)

pytestmark = pytest.mark.gpu


def fused(wl, ids=None, table=None, token_mask=None, dev_err=None):
    m = M()
    out = m.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile)
    for key in ("expand_x", "expand_scales"):
        if out.get(key) is not None:
            out[key].view(torch.uint8).fill_(POISON)
    for key in ("expert_counts", "expert_offsets", "expand_src", "assist_dst"):
        out[key].fill_(-7)
    bi = torch.full((wl.Bs, wl.K), -9, dtype=torch.int32, device="cuda")
    bm = torch.full((wl.Bs, wl.K), 7, dtype=torch.uint8, device="cuda")
    prune = wl.prune_thr is not None
    tm = wl.token_mask if token_mask is None else token_mask
    return m.moe_update_dispatch(
        cuda(wl.x), cuda(wl.logical_ids if ids is None else ids),
        cuda(wl.table if table is None else table), wl.n_ranks, wl.local_experts,
        wl.quant_mode, wl.tile, expert_scales=cuda(wl.scales) if prune else None,
        prune_thr=cuda(wl.prune_thr) if prune else None, token_mask=cuda(tm),
        balanced_ids=bi, balanced_mask=bm, out=out, dev_err=dev_err)


def check_fused(wl, ids=None, table=None, token_mask=None):
    ids_ = wl.logical_ids if ids is None else ids
    table_ = wl.table if table is None else table
    tm = wl.token_mask if token_mask is None else token_mask
    prune = wl.prune_thr is not None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = fused(wl, ids, table, token_mask, dev_err=err)
    oi, om, oe = oracle.update_expert(
        np.asarray(ids_), wl.scales.numpy() if prune else None, np.asarray(table_),
        wl.prune_thr.numpy() if prune else None, None if tm is None else np.asarray(tm), wl.E)
    np.testing.assert_array_equal(np_(g["balanced_ids"]), oi)
    np.testing.assert_array_equal(np_(g["balanced_mask"]), om)
    od = oracle_dispatch(wl, oi, om)
    total = check_dispatch(wl, g, od)
    assert int(err.item()) == (oe | od["err"])
    return g, total


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c4b"])
def test_fused_full_size(name):
    wl = W.make(name)
    say(f"[fused] {name} Bs={wl.Bs} H={wl.H} K={wl.K} E={wl.E} q={wl.quant_mode}")
    check_fused(wl)


FUSED_SMALL = [
    # seed, Bs, H, K, ranks, local, mode, tile, prune, token-mask prefix, replicas
    (201, 37, 1056, 5, 3, 4, 0, 0, True, 30, True),
    (202, 37, 1056, 5, 3, 4, 2, 0, True, None, False),
    (203, 37, 1056, 5, 3, 4, 3, 128, False, 11, True),
    (204, 37, 1056, 5, 3, 4, 4, 0, True, 36, True),
    (205, 1, 8192, 16, 128, 8, 3, 256, True, None, False),
    (206, 512, 1024, 16, 1, 16, 2, 0, True, 300, True),
    (207, 301, 7168, 8, 32, 8, 4, 0, True, 299, True),
    (208, 3, 1024, 1, 1, 1, 0, 0, False, None, False),
]


@pytest.mark.parametrize("case", FUSED_SMALL, ids=[f"f{c[0]}" for c in FUSED_SMALL])
def test_fused_small_and_edge_shapes(case):
    seed, Bs, H, K, R, L, mode, tile, prune, prefix, rep = case
    say(f"[fused] small {case}")
    wl = W.make_small(seed, Bs, H, K, R, L, mode, tile, prune=prune, shared=False,
                      token_mask_prefix=prefix, replicas=rep)
    check_fused(wl)


def test_fused_matches_separate_calls():
    wl = W.make("c4b")
    say("[fused] against the separate calls, c4b")
    g, _ = check_fused(wl)
    gi, gm = gpu_update(wl)
    gd = gpu_dispatch(wl, gi, gm)
    assert torch.equal(g["balanced_ids"], gi) and torch.equal(g["balanced_mask"], gm)
    for key in ("expert_counts", "expert_offsets", "assist_dst", "expand_src", "expand_x",
                "expand_scales"):
        assert torch.equal(g[key].view(torch.uint8), gd[key].view(torch.uint8)), key


@pytest.mark.parametrize("name", ["c4", "c4b"])
def test_single_launch_at_large_sizes(name):
    """Above 4096 entries the call runs the mapping and the dispatch as two launches when
    the mapped ids and mask are given; with them NULL it stays one launch.  Both forms give
    the same outputs and error bits (the two-launch form is checked against the oracle by
    the full-size test)."""
    m = M()
    wl = W.make(name)
    say(f"[fused] one launch against two, {name} (Bs*K = {wl.Bs * wl.K})")
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    g2 = fused(wl, dev_err=err2)
    out = m.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile)
    for key in ("expand_x", "expand_scales"):
        if out.get(key) is not None:
            out[key].view(torch.uint8).fill_(POISON)
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    prune = wl.prune_thr is not None
    t = dict(x=cuda(wl.x), ids=cuda(wl.logical_ids), table=cuda(wl.table),
             sc=cuda(wl.scales) if prune else None, thr=cuda(wl.prune_thr) if prune else None,
             tm=cuda(wl.token_mask))
    p = lambda v: None if v is None else v.data_ptr()
    n_logical, F = wl.table.shape
    rc = m.raw().moe_update_dispatch(
        p(t["x"]), p(t["ids"]), p(t["sc"]), p(t["table"]), p(t["thr"]), p(t["tm"]), wl.Bs,
        wl.H, wl.K, n_logical, F, wl.n_ranks, wl.local_experts, wl.quant_mode, wl.tile, None,
        0, None, None, p(out["expand_x"]), p(out.get("expand_scales")),
        p(out["expert_counts"]), p(out["expert_offsets"]), p(out["expand_src"]),
        p(out["assist_dst"]), p(err1), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    total = int(g2["expert_offsets"][-1].item())
    for key in ("expert_counts", "expert_offsets", "assist_dst", "expand_src"):
        assert torch.equal(out[key], g2[key]), key
    for key in ("expand_x", "expand_scales"):
        if out.get(key) is not None:
            assert torch.equal(out[key][:total].view(torch.uint8),
                               g2[key][:total].view(torch.uint8)), key
    assert int(err1.item()) == int(err2.item())


def test_fused_large_table_and_long_rows():
    """A table of 512 x 16 words (the staging limit is 8192): every block
    stages it through registers and the plain loop, and replica slots reach
    column 15."""
    rng = np.random.default_rng(2210)
    wl = W.make_small(2210, 64, 2048, 4, 16, 32, 4, 0, prune=False, shared=False)
    n_logical, F = 512, 16
    table = np.full((n_logical, F), -1, dtype=np.int32)
    for e in range(n_logical):
        n = int(rng.integers(1, F))
        table[e, 0] = n
        table[e, 1:1 + n] = rng.integers(0, wl.E, n)
    ids = rng.integers(0, n_logical, (wl.Bs, wl.K)).astype(np.int32)
    say("[fused] 512 x 16 table")
    check_fused(wl, ids=torch.from_numpy(ids), table=torch.from_numpy(table))


def test_fused_error_bits():
    wl = W.make_small(2301, 24, 1024, 4, 4, 4, 4, 0, prune=True, shared=False, replicas=True)
    say("[fused] error bits")
    ids = wl.logical_ids.clone()
    ids[2, 1] = wl.table.shape[0] + 5          # logical id out of range
    table = wl.table.clone()
    table[int(ids[5, 0]), 0] = 0               # bad replica count
    tmask = torch.ones(wl.Bs, dtype=torch.uint8)
    tmask[3] = 0                               # true, false, true...: illegal 1-D mask
    wl.scales[2, 1] = 1e30                     # keep the bad entries so their bits are raised
    wl.scales[5, 0] = 1e30
    check_fused(wl, ids=ids, table=table, token_mask=tmask)


def test_fused_rejects_a_table_too_large_to_stage():
    m = M()
    wl = W.make_small(2401, 8, 1024, 2, 2, 2, 0, 0, prune=False, shared=False)
    table = torch.from_numpy(np.tile(W.identity_table(4), (300, 7))[:1024, :9].copy())
    with pytest.raises(m.MoeError) as e:
        m.moe_update_dispatch(cuda(wl.x), cuda(wl.logical_ids), cuda(table), wl.n_ranks,
                              wl.local_experts, wl.quant_mode, wl.tile)
    assert e.value.status == m.MOE_ENOTSUP
