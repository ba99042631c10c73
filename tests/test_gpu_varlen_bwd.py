"""GPU parity of the packed variable-length backward (attn_bwd_varlen) against the fp64 oracle.
Tolerances as for the plain backward: dQ/dK/dV max-abs <= 5e-3 (fp16) / 3e-2 (bf16)."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw_varlen, round_to, varlen_lengths
from gpu_util import device, f64, to_dev
from oracle import varlen as VL

pytestmark = pytest.mark.gpu

TOL_G = {"fp16": 5e-3, "bf16": 3e-2}


def _inputs(lens, Hq, Hkv, d, dtype, seed):
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, d, seed)
    do = np.random.Generator(np.random.PCG64(seed + 1)).standard_normal(q.shape, dtype=np.float32)
    return tuple(round_to(x, dtype) for x in (q, k, v, do)) + (cu,)


def _run(q, k, v, do, cu, causal, max_seqlen):
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    tcu = torch.from_numpy(cu).to(dev)
    o, lse = eao.fwd_varlen(tq, tk, tv, tcu, max_seqlen, causal=causal)
    dq, dk, dv = eao.bwd_varlen(tq, tk, tv, o, tdo, lse, tcu, max_seqlen, causal=causal)
    torch.cuda.synchronize()
    return o, lse, f64(dq), f64(dk), f64(dv)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("fp16", 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [[1], [300], [5, 0, 129, 1, 64], [128, 127, 255, 256, 2], [700, 33]])
def test_varlen_bwd_full(dtype, d, causal, lens):
    print(f"[case] lens={lens} dtype={dtype} d={d} causal={causal}", flush=True)
    q, k, v, do, cu = _inputs(lens, 4, 2, d, dtype, seed=sum(lens) + d + 7)
    _, _, dq, dk, dv = _run(q, k, v, do, cu, causal, int(max(lens)))
    rq, rk, rv = VL.backward(q, k, v, do, cu, causal, 1.0 / np.sqrt(d))
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() <= TOL_G[dtype]


def test_varlen_bwd_equals_separate_calls():
    # each sequence's dQ is bit for bit that of attn_bwd on the sequence alone; its dK and dV are
    # the same sums up to the order of the fp32 additions (attn_bwd on one short grouped sequence
    # splits its dK/dV phase and adds the shares afterwards), compared in float32
    lens = [200, 37, 0, 512, 1]
    q, k, v, do, cu = _inputs(lens, 8, 2, 128, "bf16", seed=31)
    o, lse, dq, dk, dv = _run(q, k, v, do, cu, True, 512)
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    g32 = eao.bwd_varlen(tq, tk, tv, o, tdo, lse, torch.from_numpy(cu).to(dev), 512, causal=True,
                         grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        sl = lambda x: to_dev(x[None, :, s0:s1], dev)
        args = (sl(q), sl(k), sl(v), o[None, :, s0:s1].contiguous(), sl(do), lse[None, :, s0:s1].contiguous())
        gq, gk, gv = eao.bwd(*args, causal=True)
        sq, sk, sv = eao.bwd(*args, causal=True, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(f64(gq)[0], dq[:, s0:s1])
        assert torch.equal(sq[0], g32[0][:, s0:s1])
        for one, packed in ((sk, g32[1]), (sv, g32[2])):
            ref = f64(packed[:, s0:s1])
            assert np.abs(f64(one)[0] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max()), b


def test_varlen_bwd_larger_max_seqlen_changes_nothing():
    lens = [130, 64, 1, 250]
    q, k, v, do, cu = _inputs(lens, 4, 4, 128, "bf16", seed=41)
    a = _run(q, k, v, do, cu, True, 250)
    b = _run(q, k, v, do, cu, True, sum(lens))
    for x, y in zip(a[2:], b[2:]):
        assert np.array_equal(x, y)


def test_varlen_bwd_rows_outside_every_sequence_stay_zero():
    lens = [70, 3]
    q, k, v, do, cu = _inputs(lens + [40], 2, 1, 64, "fp16", seed=51)   # 40 trailing rows
    _, _, dq, dk, dv = _run(q, k, v, do, cu[:-1], False, 70)
    assert not dq[:, 73:].any() and not dk[:, 73:].any() and not dv[:, 73:].any()
    rq, rk, rv = VL.backward(q, k, v, do, cu[:-1], False, 1.0 / 8.0)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() <= TOL_G["fp16"]


def test_varlen_bwd_many_short_sequences_gqa():
    lens = list(varlen_lengths(64, 1, 40, seed=6))
    q, k, v, do, cu = _inputs(lens, 8, 2, 64, "fp16", seed=61)
    _, _, dq, dk, dv = _run(q, k, v, do, cu, True, int(max(lens)))
    rq, rk, rv = VL.backward(q, k, v, do, cu, True, 1.0 / 8.0)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() <= TOL_G["fp16"]


def test_varlen_bwd_packed_workload():
    # the 16-sequence packed workload (lengths in [128, 8192]): sequences the oracle finishes in
    # seconds compared element by element on two heads; every sequence checked against the
    # invariants that hold at any size (rows of P sum to 1: the dV rows of a sequence sum to its
    # dO rows summed over the query heads; rows of dS sum to 0: its dK rows sum to 0)
    lens = varlen_lengths(16, 128, 8192, seed=3)
    q, k, v, do, cu = _inputs(lens, 16, 16, 128, "bf16", seed=3)
    _, _, dq, dk, dv = _run(q, k, v, do, cu, True, int(max(lens)))
    order = np.argsort(lens)
    dof = do.to(torch.float64).numpy()
    for b in range(len(lens)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        np.testing.assert_allclose(dv[:, s0:s1].sum(axis=1), dof[:, s0:s1].sum(axis=1), atol=2e-2 * np.sqrt(s1 - s0))
        assert np.abs(dk[:, s0:s1].sum(axis=1)).max() <= 2e-2 * np.sqrt(s1 - s0)
    for b in order[:2]:
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sl = lambda x: x[:2, s0:s1]
        rq, rk, rv = VL.backward(sl(q), sl(k), sl(v), sl(do), np.array([0, s1 - s0]), True, 1.0 / np.sqrt(128))
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            assert np.abs(got[:2, s0:s1] - ref).max() <= TOL_G["bf16"]


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_float32_gradients(causal):
    """grad_dtype=float32: within the bar, and the stored bf16 gradients are these rounded."""
    lens = [300, 0, 129, 77]
    q, k, v, do, cu = _inputs(lens, 8, 2, 128, "bf16", seed=41)
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    tcu = torch.from_numpy(cu).to(dev)
    o, lse = eao.fwd_varlen(tq, tk, tv, tcu, 300, causal=causal)
    g16 = eao.bwd_varlen(tq, tk, tv, o, tdo, lse, tcu, 300, causal=causal)
    g32 = eao.bwd_varlen(tq, tk, tv, o, tdo, lse, tcu, 300, causal=causal, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = VL.backward(q, k, v, do, cu, causal, 1.0 / np.sqrt(128))
    for a, b, r in zip(g32, g16, ref):
        assert a.dtype == torch.float32
        assert torch.equal(a.to(torch.bfloat16), b)
        assert np.abs(f64(a) - r).max() <= TOL_G["bf16"]
