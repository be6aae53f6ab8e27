"""A seeded sweep of random shapes and options, each through the mapping, the
dispatch and the combine on the GPU against the oracle (the checks of
test_gpu_parity.full_chain), and through the fused mapping + dispatch
(test_gpu_fused.check_fused): token counts from 1 to 512, H from 1024 to
8192 in steps of 32, K from 1 to 16, up to 1024 instances, every quant mode
but the static one (it takes the scales input; test_gpu_scales sweeps it) with
power-of-two tiles from 16 to 1024, pruning, prefix token masks,
replicated tables and the shared expert drawn independently (and 16 draws in
the group-major mxfp8 layout).  Shapes where
Bs*K is not a multiple of 4 exercise the scalar tail of the entry loop.
"""
import numpy as np
import pytest

from combine_expert_amd import workloads as W
from tests.gpu_common import say
from tests.test_gpu_fused import check_fused
from tests.test_gpu_parity import full_chain

pytestmark = pytest.mark.gpu

N_CASES = 64
MAX_ELEMS = 1 << 25  # Bs * K * H per case, so the oracle keeps each case to seconds


def draw(seed):
    rng = np.random.default_rng(seed)
    K = int(rng.integers(1, 17))
    local = int(rng.integers(1, 17))
    ranks = int(rng.integers(1, 65))
    while ranks * local > 1024:
        ranks = max(1, ranks // 2)
    replicas = bool(rng.random() < 0.4)
    while ranks * local // (2 if replicas else 1) < K:  # enough logical experts for K
        ranks *= 2
    H = int(rng.integers(32, 257)) * 32
    Bs = int(rng.choice([1, 2, 3, 7, 31, 64, 129, 255, 300, 512]))
    while Bs > 1 and Bs * K * H > MAX_ELEMS:
        Bs //= 2
    mode = int(rng.choice([0, 2, 3, 4]))  # static mode needs the scales input: test_gpu_scales
    tile = int(2 ** rng.integers(4, 11)) if mode == W.QUANT_INT8_TILE else 128
    prune = bool(rng.random() < 0.5)
    shared = bool(rng.random() < 0.5)
    prefix = int(rng.integers(0, Bs + 1)) if rng.random() < 0.3 else None
    return dict(Bs=Bs, H=H, K=K, ranks=ranks, local=local, mode=mode, tile=tile, prune=prune,
                shared=shared, prefix=prefix, replicas=replicas)


@pytest.mark.parametrize("seed", range(900, 900 + N_CASES))
def test_random_case(seed):
    c = draw(seed)
    say(f"[sweep] {seed}: {c}")
    wl = W.make_small(seed, c["Bs"], c["H"], c["K"], c["ranks"], c["local"], c["mode"],
                      c["tile"], prune=c["prune"], shared=c["shared"],
                      token_mask_prefix=c["prefix"], replicas=c["replicas"])
    full_chain(wl)
    check_fused(wl)


@pytest.mark.parametrize("seed", range(2000, 2016))
def test_random_case_group_major_exponents(seed):
    """The same draws in the group-major mxfp8 layout (quant mode 5): H takes any multiple
    of 32, so most draws end in a partial last group of exponents."""
    c = draw(seed)
    say(f"[sweep] {seed}, group-major mxfp8: {c}")
    wl = W.make_small(seed, c["Bs"], c["H"], c["K"], c["ranks"], c["local"], 5, 128,
                      prune=c["prune"], shared=c["shared"], token_mask_prefix=c["prefix"],
                      replicas=c["replicas"])
    full_chain(wl)
    check_fused(wl)
