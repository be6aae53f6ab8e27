"""The c5 stack at its full depth: 16 chained c3-shaped layers (per layer
the mapping fused into the dispatch, int8 per token, then the combine; layer
l + 1 reads y_l as x and x_out_l as residual) captured in one HIP graph.
Every layer is checked against the oracle -- mapped ids, routing, codes and
scales bit for bit, y / x_out / rstd within tolerance -- with the oracle fed
the GPU's outputs of the layer before.  Every replay must reproduce the eager
pass bit for bit: the outputs are poisoned before each replay, other GPU work
and host synchronisation run between replays, and several replays are
checked.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import M, check_combine, np_, oracle_combine, say

pytestmark = pytest.mark.gpu

N_LAYERS = 16  # the c5 workload's depth
KEYS = ("y", "x_out", "rstd")
DKEYS = ("expand_x", "expand_scales", "expert_offsets", "assist_dst", "expand_src")


def snapshot(st):
    out = []
    for s in st["layers"]:
        out.append({k: s[k].clone() for k in KEYS} | {k: s["d"][k].clone() for k in DKEYS})
    return out


def poison(st):
    for s in st["layers"]:
        for k in KEYS:
            s[k].view(torch.uint8).fill_(0xA5)
        for k in DKEYS:
            s["d"][k].view(torch.uint8).fill_(0x5A)


def same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.fixture(scope="module")
def stack():
    m = M()
    wls = W.make_c5_layers(N_LAYERS)
    st = bench.make_stack(wls, torch, m)
    return wls, st


def test_stack_eager_against_oracle(stack):
    wls, st = stack
    m = M()
    say(f"[graph] eager {N_LAYERS}-layer stack against the oracle")
    bench.run_calls(bench.stack_calls(wls, st, m.raw(), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    x_bits = oracle.bf16_bits(wls[0].x)
    res = wls[0].residual
    for l in range(N_LAYERS):
        say(f"[graph] layer {l}")
        wl, s = wls[l], st["layers"][l]
        oi, om, _ = oracle.update_expert(wl.logical_ids.numpy(), None, wl.table.numpy(), None,
                                         None, wl.E)
        np.testing.assert_array_equal(np_(s["bal_ids"]), oi)
        od = oracle.dispatch(x_bits, oi, om, wl.n_ranks, wl.local_experts, wl.quant_mode,
                             wl.tile)
        np.testing.assert_array_equal(np_(s["d"]["assist_dst"]), od["assist"])
        total = int(od["offsets"][-1])
        np.testing.assert_array_equal(np_(s["d"]["expert_offsets"]), od["offsets"])
        np.testing.assert_array_equal(np_(s["d"]["expand_src"]), od["src"])
        gx = s["d"]["expand_x"].view(torch.uint8).cpu().numpy()[:total]
        np.testing.assert_array_equal(gx, od["expand_x"].view(np.uint8)[:total])
        gs = s["d"]["expand_scales"].cpu().numpy()[:total].reshape(-1).view(np.uint32)
        np.testing.assert_array_equal(gs, od["scales"][:total].reshape(-1).view(np.uint32))
        o = oracle_combine(wl, od["assist"], wl.expert_out, residual=res)
        check_combine((s["y"], s["x_out"], s["rstd"]), o)
        # the next layer reads this layer's GPU outputs
        x_bits = oracle.bf16_bits(s["y"].cpu())
        res = s["x_out"].cpu()


def test_graph_replays_match_eager(stack):
    wls, st = stack
    m = M()
    lib = m.raw()
    say(f"[graph] capture and replay the {N_LAYERS}-layer stack")
    bench.run_calls(bench.stack_calls(wls, st, lib, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    eager = snapshot(st)
    g = bench.capture_stack(wls, st, lib, torch)
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        poison(st)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, (s, e) in enumerate(zip(st["layers"], eager)):
            for k in KEYS:
                assert same(s[k], e[k]), (rep, l, k)
            for k in DKEYS:
                assert same(s["d"][k], e[k]), (rep, l, k)
        # unrelated eager work and an eager pass of the stack between replays
        other.mul_(1.0001).add_(0.5)
        bench.run_calls(bench.stack_calls(wls, st, lib, torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        for l, (s, e) in enumerate(zip(st["layers"], eager)):
            assert same(s["y"], e["y"]), ("eager", rep, l)
