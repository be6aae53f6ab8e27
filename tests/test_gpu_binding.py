"""The binding's dtype and size checks on CUDA tensors: a wrong dtype or an undersized
buffer raises ValueError before the library is called, so nothing is launched on it."""
import pytest
import torch

from gpu_common import M, say

pytestmark = pytest.mark.gpu


def test_wrong_dtypes_and_short_buffers_are_refused():
    m = M()
    say("[binding] argument checks")
    Bs, H, K, E = 4, 1024, 2, 8
    dev = "cuda"
    x = torch.zeros((Bs, H), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((Bs, K), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="dtype"):
        m.moe_dispatch(x.float(), ids, 1, E)
    with pytest.raises(ValueError, match="dtype"):
        m.moe_dispatch(x, ids.long(), 1, E)
    out = m.dispatch_buffers(Bs, H, K, E, m.QUANT_MXFP8, device=dev)
    out["expand_x"] = out["expand_x"][: Bs * K - 1]
    with pytest.raises(ValueError, match="expand_x"):
        m.moe_dispatch(x, ids, 1, E, quant_mode=m.QUANT_MXFP8, out=out)
    out = m.dispatch_buffers(Bs, H, K, E, m.QUANT_MXFP8, device=dev)
    out["expand_scales"] = None
    with pytest.raises(ValueError, match="expand_scales"):
        m.moe_dispatch(x, ids, 1, E, quant_mode=m.QUANT_MXFP8, out=out)
    eo = torch.zeros((Bs * K, H), dtype=torch.bfloat16, device=dev)
    s = torch.zeros((Bs, K), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="gamma"):
        m.moe_combine_add_rmsnorm(eo, ids, s, x, torch.zeros(H - 8, dtype=torch.bfloat16,
                                                             device=dev))
    with pytest.raises(ValueError, match="expert_out"):
        m.moe_combine_add_rmsnorm(eo[:-1], ids, s, x, torch.zeros(H, dtype=torch.bfloat16,
                                                                  device=dev))
    a = torch.zeros((128, H), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="^y holds"):
        m.moe_expert_gemm(a, torch.zeros((128, H // 32), dtype=torch.uint8, device=dev),
                          torch.tensor([0, 128], dtype=torch.int32, device=dev),
                          torch.zeros((1, 128, H), dtype=torch.uint8, device=dev),
                          torch.zeros((1, 2, 128, 16), dtype=torch.uint8, device=dev),
                          y=torch.zeros((127, 128), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
