"""GPU parity of the dispatch's quantisers on rows holding infinities and
NaNs, bit for bit against the oracle: per-token and per-tile int8, mxfp8 and
the static cast, without and with the scales input (one coefficient, one row
per instance), through moe_dispatch and the fused moe_update_dispatch.

The pages do not say how non-finite inputs are coded; both sides follow one
reading: a maximum skips NaN, an infinite maximum gives sharedExp 127 or the
int8 multiplier 0 with scale +inf, E4M3 codes NaN as its sign with every
other bit set and +-inf as +-448, int8 codes NaN as 0.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_expert_amd import workloads as W
from tests.gpu_common import M, POISON, check_dispatch, cuda, say

pytestmark = pytest.mark.gpu

# +inf, -inf, quiet NaN of both signs, a signalling-looking NaN, all-ones NaN
NONFINITE = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF], dtype=np.uint16)


def nonfinite_x(Bs, H, seed):
    """N(0, 1) bf16 rows: in every third row about 1 element in 150 is replaced
    by an infinity or a NaN, in the next about 1 in 300 by a NaN only, and the
    third stays finite (so per-token maxima are infinite, finite beside NaN,
    and finite).  Hand-placed cases on top: a block of NaN only, a block with
    an infinity beside the largest finite values, a block whose only
    non-finite element is a NaN, a row of NaN only and a row with a single
    -inf."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((Bs, H)).astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any finite bf16 will do
    u = rng.random((Bs, H))
    kind = (np.arange(Bs) % 3)[:, None]
    hit = (kind == 0) & (u < 1.0 / 150)
    b[hit] = rng.choice(NONFINITE, size=int(hit.sum()))
    hit = (kind == 1) & (u < 1.0 / 300)
    b[hit] = rng.choice(NONFINITE[2:], size=int(hit.sum()))
    b[0, :32] = 0x7FC0
    b[1, 32:64] = rng.choice(np.array([0x7A00, 0x7A80, 0x7F7F, 0xFF7F, 0x3F80], np.uint16), 32)
    b[1, 40] = 0x7F80
    b[2, 64:96] = (f[2, 64:96].view(np.uint32) >> 16).astype(np.uint16)
    b[2, 70] = 0xFFC0
    if Bs > 4:
        b[3, :] = 0x7FC0
        b[4, :] = (f[4].view(np.uint32) >> 16).astype(np.uint16)
        b[4, H // 2] = 0xFF80
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)


def run(wl, qs, kind, fused):
    m = M()
    out = m.dispatch_buffers(wl.Bs, wl.H, wl.K, wl.E, wl.quant_mode, wl.tile)
    for key in ("expand_x", "expand_scales"):
        if out.get(key) is not None:
            out[key].view(torch.uint8).fill_(POISON)
    for key in ("expert_counts", "expert_offsets", "expand_src", "assist_dst"):
        out[key].fill_(-7)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if fused:
        out = m.moe_update_dispatch(cuda(wl.x), cuda(wl.logical_ids), cuda(wl.table), wl.n_ranks,
                                    wl.local_experts, wl.quant_mode, wl.tile,
                                    quant_scales=cuda(qs), out=out, dev_err=err)
    else:
        out = m.moe_dispatch(cuda(wl.x), cuda(wl.logical_ids), wl.n_ranks, wl.local_experts,
                             wl.quant_mode, wl.tile, quant_scales=cuda(qs), out=out, dev_err=err)
    od = oracle.dispatch(oracle.bf16_bits(wl.x), wl.logical_ids.numpy(), None, wl.n_ranks,
                         wl.local_experts, wl.quant_mode, wl.tile,
                         None if qs is None else qs.numpy(), kind)
    check_dispatch(wl, out, od)
    assert int(err.item()) == int(od["err"])


CASES = [
    # seed, Bs, H, K, ranks, local, mode, tile, scales kind, fused
    (401, 37, 2080, 4, 2, 4, 2, 0, 0, False),
    (402, 37, 2080, 4, 2, 4, 3, 32, 0, False),
    (403, 37, 4128, 4, 2, 4, 3, 128, 0, False),
    (404, 37, 2080, 4, 2, 4, 4, 0, 0, False),
    (405, 64, 7168, 8, 4, 8, 4, 0, 0, True),
    (406, 19, 1056, 3, 2, 3, 1, 0, 1, False),
    (407, 19, 1056, 3, 2, 3, 1, 0, 3, False),
    (408, 19, 2080, 3, 2, 3, 2, 0, 3, False),
    (409, 19, 2080, 3, 2, 3, 3, 128, 3, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}" for c in CASES])
def test_quantisers_on_nonfinite_rows(case):
    seed, Bs, H, K, R, L, mode, tile, kind, fused = case
    say(f"[nonfinite] {case}")
    wl = W.make_small(seed, Bs, H, K, R, L, mode, tile, shared=False)
    wl.x = nonfinite_x(Bs, H, seed)
    qs = W.make_quant_scales(seed, kind, wl.E, wl.H)
    run(wl, qs, kind, fused)
