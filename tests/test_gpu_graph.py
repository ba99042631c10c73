"""The entry points under HIP graph capture (torch.cuda.CUDAGraph, which records what is launched
on torch's current stream): the library only launches kernels (it allocates, clears and waits for
nothing), so a captured forward + backward, variable-length forward + backward and split-KV decode
replay to the eager results bit for bit.  New inputs are copied in before each of several replays,
with eager calls and synchronisations between them, and every replay is checked."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, draw_decode, draw_varlen, round_to
from gpu_util import device, f64
from oracle import attention as A

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _static(shapes_dtype, dev):
    return [torch.empty(s, dtype=dt, device=dev) for s, dt in shapes_dtype]


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                    # eager call on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_dense_fwd_bwd():
    dev = device()
    B, Hq, Hkv, N, d, causal = 1, 4, 2, 515, 128, True
    q, k, v, do = _static([((B, Hq, N, d), torch.bfloat16), ((B, Hkv, N, d), torch.bfloat16),
                           ((B, Hkv, N, d), torch.bfloat16), ((B, Hq, N, d), torch.bfloat16)], dev)
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = torch.empty(eao.bwd_workspace_size(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)

    def step():
        eao.fwd(q, k, v, causal=causal, out=o, lse=lse)
        eao.bwd(q, k, v, o, do, lse, causal=causal, workspace=ws, dq=dq, dk=dk, dv=dv)

    for x, y in zip((q, k, v, do), draw(B, Hq, Hkv, N, d, 900, with_grad=True)[1:]):
        x.copy_(round_to(y, "bf16"))
    g = _capture(step)
    for r in range(REPLAYS):
        host = [round_to(y, "bf16") for y in draw(B, Hq, Hkv, N, d, 901 + r, with_grad=True)[1:]]
        for x, y in zip((q, k, v, do), host):
            x.copy_(y)
        g.replay()
        torch.cuda.synchronize()
        eo, el = eao.fwd(q, k, v, causal=causal)
        edq, edk, edv = eao.bwd(q, k, v, eo, do, el, causal=causal)
        torch.cuda.synchronize()
        for got, want in ((o, eo), (lse, el), (dq, edq), (dk, edk), (dv, edv)):
            assert torch.equal(got, want), r
        if r == REPLAYS - 1:
            ro, _ = A.forward(*host[:3], causal, 1.0 / np.sqrt(d))
            assert np.abs(f64(o) - ro).max() <= 1.5e-2


def test_graph_varlen_fwd_bwd():
    dev = device()
    lens, Hq, Hkv, d, causal = [200, 1, 0, 333, 64], 4, 2, 128, True
    ms = max(lens)
    q0, k0, v0, cu = draw_varlen(lens, Hq, Hkv, d, 910)
    T = q0.shape[1]
    q, do = torch.empty((Hq, T, d), dtype=torch.bfloat16, device=dev), torch.empty((Hq, T, d), dtype=torch.bfloat16, device=dev)
    k, v = torch.empty((Hkv, T, d), dtype=torch.bfloat16, device=dev), torch.empty((Hkv, T, d), dtype=torch.bfloat16, device=dev)
    tcu = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ws = torch.empty(max(eao.bwd_varlen_workspace_size(len(lens), Hq, Hkv, ms, d), 1), dtype=torch.uint8, device=dev)

    def fill(seed):
        a, b, c, _ = draw_varlen(lens, Hq, Hkv, d, seed)
        g = np.random.Generator(np.random.PCG64(seed + 1)).standard_normal(a.shape, dtype=np.float32)
        for x, y in zip((q, k, v, do), (a, b, c, g)):
            x.copy_(round_to(y, "bf16"))

    def step():
        eao.fwd_varlen(q, k, v, tcu, ms, causal=causal, out=o, lse=lse)
        eao.bwd_varlen(q, k, v, o, do, lse, tcu, ms, causal=causal, workspace=ws, dq=dq, dk=dk, dv=dv)

    fill(910)
    g = _capture(step)
    for r in range(REPLAYS):
        fill(911 + 2 * r)
        g.replay()
        torch.cuda.synchronize()
        eo, el = eao.fwd_varlen(q, k, v, tcu, ms, causal=causal)
        edq, edk, edv = eao.bwd_varlen(q, k, v, eo, do, el, tcu, ms, causal=causal)
        torch.cuda.synchronize()
        for got, want in ((o, eo), (lse, el), (dq, edq), (dk, edk), (dv, edv)):
            assert torch.equal(got, want), r


def test_graph_splitkv_decode():
    dev = device()
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 1, 3000, 128
    q0, k0, v0 = draw_decode(B, Hq, Hkv, Nq, Nk, d, 920)[:3]
    q = torch.empty(tuple(q0.shape), dtype=torch.bfloat16, device=dev)
    k = torch.empty(tuple(k0.shape), dtype=torch.bfloat16, device=dev)
    v = torch.empty(tuple(v0.shape), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(eao.splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d), 256), dtype=torch.uint8, device=dev)

    def fill(seed):
        for x, y in zip((q, k, v), draw_decode(B, Hq, Hkv, Nq, Nk, d, seed)[:3]):
            x.copy_(round_to(y, "bf16"))

    def step():
        eao.fwd_splitkv(q, k, v, causal=True, workspace=ws, out=o, lse=lse)

    fill(920)
    g = _capture(step)
    for r in range(REPLAYS):
        fill(921 + r)
        g.replay()
        torch.cuda.synchronize()
        eo, el = eao.fwd_splitkv(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), r
