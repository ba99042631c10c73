"""GPU parity of the backward with a sliding window and/or ALiBi (attn_bwd_ext) against the fp64
oracle.  Tolerances as for the plain backward: dQ/dK/dV max-abs <= 5e-3 (fp16) / 3e-2 (bf16)."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, round_to
from gpu_util import device, f64, to_dev
from oracle import variants as VA

pytestmark = pytest.mark.gpu

TOL_G = {"fp16": 5e-3, "bf16": 3e-2}


def _inputs(B, Hq, Hkv, N, d, dtype, seed):
    _, q, k, v, do = draw(B, Hq, Hkv, N, d, seed, with_grad=True)
    return tuple(round_to(x, dtype) for x in (q, k, v, do))


def _slopes(Hq):
    return (2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq)).astype(np.float32)


def _run(q, k, v, do, causal, window, slopes):
    dev = device()
    ts = None if slopes is None else torch.from_numpy(slopes).to(dev)
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    o, lse = eao.fwd_ext(tq, tk, tv, causal=causal, window=window, alibi_slopes=ts)
    dq, dk, dv = eao.bwd_ext(tq, tk, tv, o, tdo, lse, causal=causal, window=window, alibi_slopes=ts)
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,window", [(1, 1), (63, 16), (200, 1), (200, 64), (515, 100), (515, 128), (300, 1000)])
@pytest.mark.parametrize("alibi", [False, True])
def test_bwd_ext_small_full(dtype, d, causal, N, window, alibi):
    print(f"[case] N={N} window={window} alibi={alibi} dtype={dtype} d={d} causal={causal}", flush=True)
    B, Hq, Hkv = 2, 4, 2
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, dtype, seed=N + window + d + 1)
    sl = _slopes(Hq) if alibi else None
    got = _run(q, k, v, do, causal, window, sl)
    ref = VA.backward(q, k, v, do, causal, 1.0 / np.sqrt(d), window=window, slopes=sl)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= TOL_G[dtype]


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ext_alibi_only_gqa(causal):
    q, k, v, do = _inputs(1, 8, 2, 777, 128, "bf16", seed=13)
    sl = _slopes(8)
    got = _run(q, k, v, do, causal, 0, sl)
    ref = VA.backward(q, k, v, do, causal, 1.0 / np.sqrt(128), slopes=sl)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= TOL_G["bf16"]


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ext_without_window_or_bias_matches_attn_bwd(causal):
    q, k, v, do = _inputs(1, 4, 4, 333, 128, "bf16", seed=14)
    got = _run(q, k, v, do, causal, 0, None)
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    o, lse = eao.fwd(tq, tk, tv, causal=causal)
    ref = eao.bwd(tq, tk, tv, o, tdo, lse, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert np.abs(a - f64(b)).max() <= TOL_G["bf16"] / 8


def test_bwd_ext_medium_window_alibi():
    # several key blocks and query blocks inside and across the band, causal, N not a tile multiple
    q, k, v, do = _inputs(1, 4, 4, 2111, 128, "bf16", seed=15)
    sl = _slopes(4)
    got = _run(q, k, v, do, True, 300, sl)
    ref = VA.backward(q, k, v, do, True, 1.0 / np.sqrt(128), window=300, slopes=sl)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= TOL_G["bf16"]


def test_bwd_ext_long_workload_invariants():
    # the long shape with a 4096-key window and ALiBi (the forward's window/ALiBi workload): rows
    # of P sum to 1, so the dV rows of a head sum to its dO rows; rows of dS sum to 0, so the dK
    # rows sum to 0
    q, k, v, do = _inputs(1, 16, 16, 16384, 128, "bf16", seed=3)
    got = _run(q, k, v, do, True, 4096, _slopes(16))
    dq, dk, dv = got
    for x in got:
        assert np.isfinite(x).all()
    dof = do.to(torch.float64).numpy()
    np.testing.assert_allclose(dv[0].sum(axis=1), dof[0].sum(axis=1), atol=2.0)
    assert np.abs(dk[0].sum(axis=1)).max() <= 2.0


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ext_float32_gradients(causal):
    """grad_dtype=float32: the accumulators unrounded, within the bar; rounded, the bf16 result."""
    q, k, v, do = _inputs(2, 8, 2, 400, 128, "bf16", seed=15)
    sl = _slopes(8)
    dev = device()
    ts = torch.from_numpy(sl).to(dev)
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    o, lse = eao.fwd_ext(tq, tk, tv, causal=causal, window=150, alibi_slopes=ts)
    g16 = eao.bwd_ext(tq, tk, tv, o, tdo, lse, causal=causal, window=150, alibi_slopes=ts)
    g32 = eao.bwd_ext(tq, tk, tv, o, tdo, lse, causal=causal, window=150, alibi_slopes=ts, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = VA.backward(q, k, v, do, causal, 1.0 / np.sqrt(128), window=150, slopes=sl)
    for a, b, r in zip(g32, g16, ref):
        assert a.dtype == torch.float32
        assert torch.equal(a.to(torch.bfloat16), b)
        assert np.abs(f64(a) - r).max() <= TOL_G["bf16"]
