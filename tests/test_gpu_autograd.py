"""The differentiable op: gradients through torch autograd equal attn_bwd's bit for bit and the
fp64 oracle's within the backward tolerances."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, round_to
from gpu_util import device, f64, to_dev
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL = {"fp16": 5e-3, "bf16": 3e-2}


@pytest.mark.parametrize("dtype,Hq,Hkv,N,causal", [("bf16", 4, 2, 300, True), ("fp16", 2, 2, 129, False)])
def test_autograd_matches_attn_bwd_and_oracle(dtype, Hq, Hkv, N, causal):
    _, q, k, v, do = draw(1, Hq, Hkv, N, 128, seed=N + Hq, with_grad=True)
    qc, kc, vc, doc = (round_to(x, dtype) for x in (q, k, v, do))
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (qc, kc, vc, doc))
    lq, lk, lv = (t.clone().requires_grad_() for t in (tq, tk, tv))
    o = eao.attention(lq, lk, lv, causal=causal)
    o.backward(tdo)
    o2, lse = eao.fwd(tq, tk, tv, causal=causal)
    dq, dk, dv = eao.bwd(tq, tk, tv, o2, tdo, lse, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b in ((lq.grad, dq), (lk.grad, dk), (lv.grad, dv)):
        assert torch.equal(a, b)
    refs = A.backward(qc, kc, vc, doc, causal, 1.0 / np.sqrt(128))
    for a, r in zip((lq.grad, lk.grad, lv.grad), refs):
        assert np.abs(f64(a) - r).max() <= TOL[dtype]
