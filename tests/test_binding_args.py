"""The binding checks tensor arguments before their pointers reach the library (host
only): host tensors are refused with ValueError, so no kernel is ever handed a host
address.  The dtype and size checks need CUDA tensors and are covered by a GPU test."""
import pytest
import torch

from combine_expert_amd import moe


def test_host_tensors_are_refused():
    Bs, H, K, E = 4, 1024, 2, 8
    x = torch.zeros((Bs, H), dtype=torch.bfloat16)
    ids = torch.zeros((Bs, K), dtype=torch.int32)
    table = torch.ones((E, 2), dtype=torch.int32)
    out = moe.dispatch_buffers(Bs, H, K, E, moe.QUANT_NONE, device="cpu")
    with pytest.raises(ValueError, match="CUDA"):
        moe.moe_dispatch(x, ids, 1, E, out=out, stream=0)
    with pytest.raises(ValueError, match="CUDA"):
        moe.moe_update_expert(ids, table, E, stream=0)
    with pytest.raises(ValueError, match="CUDA"):
        moe.moe_update_dispatch(x, ids, table, 1, E, out=out, balanced_ids=ids.clone(),
                                balanced_mask=torch.zeros((Bs, K), dtype=torch.uint8), stream=0)
    eo = torch.zeros((Bs * K, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="CUDA"):
        moe.moe_combine_add_rmsnorm(eo, ids, torch.zeros((Bs, K)), x, torch.zeros(H, dtype=torch.bfloat16),
                                    y=x.clone(), x_out=x.clone(), rstd=torch.zeros(Bs), stream=0)
    a = torch.zeros((128, H), dtype=torch.uint8)
    with pytest.raises(ValueError, match="CUDA"):
        moe.moe_expert_gemm(a, torch.zeros((128, H // 32), dtype=torch.uint8),
                            torch.tensor([0, 128], dtype=torch.int32),
                            torch.zeros((1, 128, H), dtype=torch.uint8),
                            torch.zeros((1, 2, 128, 16), dtype=torch.uint8),
                            y=torch.zeros((128, 128), dtype=torch.bfloat16), stream=0)
