"""The allocation-free split-KV entry point (attn_fwd_splitkv_noalloc), for callers that cannot
allocate: its partials live in the library's static per-GPU scratch buffer.  Through the C ABI it
must give exactly what attn_fwd_splitkv (same kernels, caller's workspace) gives, on two calls in
a row, the second smaller (whatever the first left in the buffer), and reject a problem whose
partials exceed the buffer before launching anything."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw_decode, round_to
from gpu_util import device, f64, to_dev
from oracle import decode as DC

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed, dev):
    q, k, v = draw_decode(B, Hq, Hkv, Nq, Nk, d, seed)
    return tuple(to_dev(round_to(x, dtype), dev) for x in (q, k, v))


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    dev = device()
    cases = [  # B, Hq, Hkv, Nq, Nk, d, dtype, causal, splits: the second smaller than the first
        (4, 32, 8, 2, 8192, 128, "bf16", True, 0),
        (2, 8, 2, 3, 1000, 64, "fp16", True, 3),
    ]
    for i, (B, Hq, Hkv, Nq, Nk, d, dtype, causal, splits) in enumerate(cases):
        print(f"[case] noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype}", flush=True)
        assert eao.splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, splits) <= (8 << 20)
        q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, 40 + i, dev)
        o_ref, l_ref = eao.fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
        eao.fwd_splitkv_noalloc(q, k, v, o, lse, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), i
        # and the result is the attention itself (one query head, against the oracle)
        ro, rlse = DC.forward(q[:1, :1].cpu(), k[:1, :1].cpu(), v[:1, :1].cpu(), causal, 1.0 / np.sqrt(d))
        tol = {"bf16": 1.5e-2, "fp16": 2e-3}[dtype]
        assert np.abs(f64(o[:1, :1]) - ro).max() <= tol
        assert np.abs(f64(lse[:1, :1]) - rlse).max() <= 1e-3


def test_noalloc_rejects_problems_beyond_its_scratch():
    dev = device()
    q = torch.zeros(16, 64, 64, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(16, 64, 4096, 128, dtype=torch.bfloat16, device=dev)
    o, lse = torch.empty_like(q), torch.empty(16, 64, 64, dtype=torch.float32, device=dev)
    assert eao.splitkv_workspace_size(16, 64, 64, 64, 4096, 128, 0) > (8 << 20)
    with pytest.raises(eao.AttnError, match="scratch"):
        eao.fwd_splitkv_noalloc(q, k, k, o, lse, causal=True)
