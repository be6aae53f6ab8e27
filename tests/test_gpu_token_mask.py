"""The dispatch's 1-D active mask ("aclnnMoeDistributeDispatchV2", 参数说明:
the active mask may be given per token, shape (Bs,), or per entry, (Bs, K)).
An entry is active only if both masks given allow it, so the GPU output must
equal the oracle's dispatch run with the per-entry mask that the two make
together (composed here with numpy).  A per-token mask that is not all true,
then all false raises error bit 4 and is still applied as given.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import M, check_dispatch, cuda, np_, say

pytestmark = pytest.mark.gpu


def run(wl, tok, mask2d):
    m = M()
    out = m.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile)
    for key in ("expand_x", "expand_scales"):
        if out.get(key) is not None:
            out[key].view(torch.uint8).fill_(0xAB)
    for key in ("expert_counts", "expert_offsets", "expand_src", "assist_dst"):
        out[key].fill_(-7)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = m.moe_dispatch(cuda(wl.x), cuda(wl.logical_ids), wl.n_ranks, wl.local_experts,
                       wl.quant_mode, wl.tile,
                       active_mask=None if mask2d is None else torch.from_numpy(mask2d).cuda(),
                       token_mask=torch.from_numpy(tok).cuda(), out=out, dev_err=err)
    both = np.repeat(tok[:, None].astype(np.uint8), wl.K, axis=1)
    if mask2d is not None:
        both = both & mask2d
    o = oracle.dispatch(oracle.bf16_bits(wl.x), wl.logical_ids.numpy(), both, wl.n_ranks,
                        wl.local_experts, wl.quant_mode, wl.tile)
    check_dispatch(wl, g, o)
    return int(err.item())


CASES = [  # (seed, Bs, H, K, ranks, local, quant, tile)
    (11, 64, 2048, 4, 4, 4, W.QUANT_MXFP8, 0),
    (12, 96, 1024, 8, 8, 8, W.QUANT_INT8_TOKEN, 0),
    (13, 40, 4096, 6, 5, 3, W.QUANT_INT8_TILE, 128),
    (14, 33, 1056, 3, 2, 4, W.QUANT_NONE, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_prefix_token_mask(case):
    seed, Bs, H, K, R, L, q, tile = case
    say(f"[token mask] prefix {case}")
    wl = W.make_small(seed=seed, Bs=Bs, H=H, K=K, n_ranks=R, local_experts=L, quant_mode=q)
    wl.tile = tile
    tok = np.zeros(Bs, dtype=np.uint8)
    tok[: Bs * 2 // 3] = 1
    assert run(wl, tok, None) == 0
    rng = np.random.default_rng(seed)
    mask2d = (rng.random((Bs, K)) < 0.7).astype(np.uint8)
    assert run(wl, tok, mask2d) == 0
    assert run(wl, np.ones(Bs, np.uint8), None) == 0
    assert run(wl, np.zeros(Bs, np.uint8), None) == 0


def test_illegal_token_mask_raises_bit4_and_is_applied():
    say("[token mask] {true, false, true}")
    wl = W.make_small(seed=21, Bs=48, H=2048, K=4, n_ranks=4, local_experts=4,
                      quant_mode=W.QUANT_MXFP8)
    tok = np.ones(48, dtype=np.uint8)
    tok[10] = 0
    assert run(wl, tok, None) & 4
