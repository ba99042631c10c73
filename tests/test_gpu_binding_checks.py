"""On the GPU: caller-supplied outputs, gradients, workspaces and offsets that are host tensors,
or of the wrong shape or dtype, are rejected by the binding before any kernel is launched."""
import pytest
import torch

import exact_attention_online_amd as eao
from gpu_util import device

pytestmark = pytest.mark.gpu


def _qkv(dev, B=1, H=2, N=64, d=64):
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    return q, q.clone(), q.clone()


def test_fwd_rejects_host_or_misshapen_outputs():
    dev = device()
    q, k, v = _qkv(dev)
    with pytest.raises(eao.AttnError, match="out"):
        eao.fwd(q, k, v, out=torch.empty_like(q, device="cpu"))
    with pytest.raises(eao.AttnError, match="lse"):
        eao.fwd(q, k, v, lse=torch.empty(1, 2, 64))
    with pytest.raises(eao.AttnError, match="lse"):
        eao.fwd(q, k, v, lse=torch.empty(1, 2, 63, device=dev))
    with pytest.raises(eao.AttnError, match="out"):
        eao.fwd(q, k, v, out=torch.empty(q.shape, dtype=torch.float16, device=dev))


def test_bwd_rejects_host_or_misshapen_arguments():
    dev = device()
    q, k, v = _qkv(dev)
    o, lse = eao.fwd(q, k, v)
    do = torch.zeros_like(q)
    torch.cuda.synchronize()
    with pytest.raises(eao.AttnError, match="do"):
        eao.bwd(q, k, v, o, do.cpu(), lse)
    with pytest.raises(eao.AttnError, match="lse"):
        eao.bwd(q, k, v, o, do, lse.cpu())
    with pytest.raises(eao.AttnError, match="workspace"):
        eao.bwd(q, k, v, o, do, lse, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(eao.AttnError, match="dq"):
        eao.bwd(q, k, v, o, do, lse, dq=torch.empty_like(q, device="cpu"))
    with pytest.raises(eao.AttnError, match="dk"):
        eao.bwd(q, k, v, o, do, lse, dk=torch.empty(1, 2, 64, 32, dtype=torch.bfloat16, device=dev))
    with pytest.raises(eao.AttnError, match="grad_dtype"):
        eao.bwd(q, k, v, o, do, lse, grad_dtype=torch.float16)
    # float32 gradients need float32 outputs
    with pytest.raises(eao.AttnError, match="dq"):
        eao.bwd(q, k, v, o, do, lse, grad_dtype=torch.float32, dq=torch.empty_like(q))


def test_varlen_rejects_host_offsets_and_outputs():
    dev = device()
    q = torch.zeros(2, 100, 64, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=dev)
    with pytest.raises(eao.AttnError):
        eao.fwd_varlen(q, q, q, cu.cpu(), 60)
    with pytest.raises(eao.AttnError, match="out"):
        eao.fwd_varlen(q, q, q, cu, 60, out=torch.empty_like(q, device="cpu"))
    o, lse = eao.fwd_varlen(q, q, q, cu, 60)
    torch.cuda.synchronize()
    with pytest.raises(eao.AttnError, match="lse"):
        eao.bwd_varlen(q, q, q, o, q, lse.cpu(), cu, 60)
