"""Tensors past 2^31 elements: B=1, H=1040, N=16384, d=128 bf16 (4.4 GB per tensor), causal, so
that heads 1024 and up start beyond 2^31 elements (4 GiB) of Q, K, V, O, dO, dQ, dK, dV and of
the backward's workspace.  The forward is checked on sampled rows of heads on both sides of that
boundary and of the last head, the backward on one whole head past it, against the fp64 oracle,
with the tolerances of the other parity tests (O 1.5e-2, LSE 1e-3, gradients 3e-2 for bf16)."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw_on_device
from gpu_util import device, f64, sample_rows
from oracle import attention as A

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 1040, 16384, 128


def test_beyond_2_31_elements_fwd_bwd():
    dev = device()
    assert B * H * N * D > 2**31
    print(f"[case] B={B} H={H} N={N} d={D} bf16 causal", flush=True)
    q, k, v, do = draw_on_device([(B, H, N, D)] * 4, "bf16", 31, dev)
    o, lse = eao.fwd(q, k, v, causal=True)
    dq, dk, dv = eao.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    rows = sample_rows(N, n_random=24, seed=31)
    ri = torch.from_numpy(rows).to(dev)
    for h in (1023, 1024, H - 1):
        print(f"  oracle forward rows of head {h}", flush=True)
        hq, hk, hv = (x[:, h:h + 1].cpu() for x in (q, k, v))
        ro, rl = A.forward_rows(hq, hk, hv, True, scale, 0, 0, rows)
        assert np.abs(f64(o[0, h].index_select(0, ri)) - ro).max() <= 1.5e-2, h
        assert np.abs(f64(lse[0, h].index_select(0, ri)) - rl).max() <= 1e-3, h
    h = 1024
    print(f"  oracle backward of head {h}", flush=True)
    hq, hk, hv, hdo = (x[:, h:h + 1].cpu() for x in (q, k, v, do))
    rq, rk, rv, _ = A.backward_group(hq, hk, hv, hdo, True, scale, 0, 0, row_block=1024)
    assert np.abs(f64(dq[0, h]) - rq[0]).max() <= 3e-2
    assert np.abs(f64(dk[0, h]) - rk).max() <= 3e-2
    assert np.abs(f64(dv[0, h]) - rv).max() <= 3e-2
    for t in (o, lse, dq[0, H - 1], dk[0, H - 1], dv[0, H - 1]):
        assert torch.isfinite(t).all()
