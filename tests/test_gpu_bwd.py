"""GPU parity of the backward kernels against the fp64 oracle (through the C ABI).

Tolerances (max-abs over every compared element): dQ, dK, dV <= 5e-3 for fp16 and <= 3e-2 for
bf16 on unit-normal inputs.  The GPU backward consumes the GPU forward's O and LSE (the real
pipeline); one case feeds the oracle's O and LSE instead to isolate the backward kernels.
Small problems are compared over every output; the large workloads over whole K/V head groups
(every dK/dV row of the group and every dQ row of its query heads).
"""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import WORKLOADS, draw, round_to
from gpu_util import device, f64, to_dev
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL = {"fp16": 5e-3, "bf16": 3e-2}


def _inputs(B, Hq, Hkv, N, d, dtype, seed):
    _, q, k, v, do = draw(B, Hq, Hkv, N, d, seed, with_grad=True)
    return [round_to(x, dtype) for x in (q, k, v, do)]


def _gpu_grads(q, k, v, do, causal, scale=None, o=None, lse=None):
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    if o is None:
        o, lse = eao.fwd(tq, tk, tv, causal=causal, scale=scale)
    else:
        o, lse = to_dev(o, dev), to_dev(lse, dev)
    dq, dk, dv = eao.bwd(tq, tk, tv, o, tdo, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _err(gpu, ref):
    return float(np.abs(f64(gpu) - ref).max())


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 127, 129, 200, 515])
def test_backward_small_full(dtype, d, causal, N):
    q, k, v, do = _inputs(1, 4, 2, N, d, dtype, seed=N * 3 + d + causal)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal)
    rq, rk, rv = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(d))
    assert _err(dq, rq) <= TOL[dtype]
    assert _err(dk, rk) <= TOL[dtype]
    assert _err(dv, rv) <= TOL[dtype]


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_gqa_full(Hq, Hkv, causal):
    q, k, v, do = _inputs(2, Hq, Hkv, 300, 128, "bf16", seed=100 + Hq * 10 + Hkv)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal)
    rq, rk, rv = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(128))
    assert _err(dq, rq) <= TOL["bf16"]
    assert _err(dk, rk) <= TOL["bf16"]
    assert _err(dv, rv) <= TOL["bf16"]


def test_backward_with_oracle_forward_outputs():
    """Isolate the backward kernels: O and LSE come from the oracle (O rounded to bf16)."""
    N, d = 333, 128
    q, k, v, do = _inputs(1, 2, 2, N, d, "bf16", seed=77)
    ro, rlse = A.forward(q, k, v, True, 1.0 / np.sqrt(d))
    o = torch.from_numpy(ro).to(torch.bfloat16)
    lse = torch.from_numpy(rlse).to(torch.float32)
    dq, dk, dv = _gpu_grads(q, k, v, do, True, o=o, lse=lse)
    rq, rk, rv = A.backward(q, k, v, do, True, 1.0 / np.sqrt(d))
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        assert _err(g, r) <= TOL["bf16"]


def test_custom_scale_fp16():
    q, k, v, do = _inputs(1, 2, 1, 150, 64, "fp16", seed=78)
    dq, dk, dv = _gpu_grads(q, k, v, do, False, scale=0.07)
    rq, rk, rv = A.backward(q, k, v, do, False, 0.07)
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        assert _err(g, r) <= TOL["fp16"]


def _group_check(w, seed, groups, row_block):
    q, k, v, do = _inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, seed=seed)
    dq, dk, dv = _gpu_grads(q, k, v, do, w.causal)
    G = w.Hq // w.Hkv
    for b, g in groups:
        print(f"  oracle group b={b} g={g}", flush=True)
        rq, rk, rv, _ = A.backward_group(q, k, v, do, w.causal, w.scale, b, g, row_block=row_block)
        assert _err(dk[b, g], rk) <= TOL[w.dtype], ("dk", b, g)
        assert _err(dv[b, g], rv) <= TOL[w.dtype], ("dv", b, g)
        assert _err(dq[b, g * G:(g + 1) * G], rq) <= TOL[w.dtype], ("dq", b, g)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


def test_gqa_workload_groups():
    _group_check(WORKLOADS["gqa_bf16"], 4, [(0, 0), (3, 7)], row_block=1024)


def test_long_workload_one_head():
    _group_check(WORKLOADS["long_bf16"], 3, [(0, 5)], row_block=1024)


# ---------------------------------------------------------------- invariants on the device
def test_gradient_sums():
    """sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 per head (rows of P sum to 1, of dS to 0)."""
    q, k, v, do = _inputs(1, 2, 2, 700, 128, "fp16", seed=79)
    dq, dk, dv = _gpu_grads(q, k, v, do, True)
    np.testing.assert_allclose(f64(dv).sum(2), f64(do).sum(2), atol=0.05)
    assert np.abs(f64(dk).sum(2)).max() <= 0.05


def test_gradients_deterministic():
    q, k, v, do = _inputs(1, 4, 2, 600, 128, "bf16", seed=80)
    g1 = _gpu_grads(q, k, v, do, True)
    g2 = _gpu_grads(q, k, v, do, True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_workspace_contents_do_not_matter():
    q, k, v, do = _inputs(1, 2, 2, 260, 128, "bf16", seed=81)
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    o, lse = eao.fwd(tq, tk, tv, causal=True)
    ws = torch.full((eao.bwd_workspace_size(1, 2, 2, 260, 128),), 0x7F, dtype=torch.uint8, device=dev)
    a = eao.bwd(tq, tk, tv, o, tdo, lse, causal=True, workspace=ws)
    b = eao.bwd(tq, tk, tv, o, tdo, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert _err(x, f64(y)) <= 1e-2


@pytest.mark.parametrize("kind", ["up", "down", "spike"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_running_maximum_growth(kind, dtype, causal):
    # inputs of test_gpu_fwd's running-maximum test (scores up to about 100); the gradients scale
    # with |K| and |Q| (about 30-40 along one direction), so the bar is the unit-normal one
    # relative to max(1, max |reference|)
    from test_gpu_fwd import _ramp_inputs

    q, k, v = _ramp_inputs(kind, 515, 128, dtype, seed=12)
    g = np.random.Generator(np.random.PCG64(13))
    do = round_to(g.standard_normal(q.shape, dtype=np.float32), dtype)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal)
    refs = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(128))
    for got, ref in zip((dq, dk, dv), refs):
        assert _err(got, ref) <= TOL[dtype] * max(1.0, np.abs(ref).max())


# ---------------------------------------------------------------- dQ block size chosen by grid size
# The dQ kernel takes 256-row blocks (8 waves) when B*Hq*ceil(N/256) >= 512, else 128-row blocks
# (4 waves).  Below: 4*64*ceil(300/256) = 512 blocks, so the 8-wave path, over every output with a
# ragged tail (300 = 256 + 44); one head alone takes the 4-wave path, and a row's arithmetic is the
# same in both, so its dQ agrees bit for bit.  One query head per K/V head: grouped sums are covered
# above; summed over 4 heads, dK reaches |4..8| where a bf16 step is 0.0156, and over the 2.4M
# outputs of this shape the largest grouped dK error came to 0.034, past the absolute bar.
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_grid_full_and_block_size_invariance(dtype, d, causal):
    B, Hq, Hkv, N = 4, 64, 64, 300
    assert B * Hq * ((N + 255) // 256) >= 512
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, dtype, seed=90 + d + causal)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal)
    rq, rk, rv = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(d))
    assert _err(dq, rq) <= TOL[dtype]
    assert _err(dk, rk) <= TOL[dtype]
    assert _err(dv, rv) <= TOL[dtype]
    G = Hq // Hkv
    for b, h in ((0, 0), (2, 37), (3, 63)):
        g = h // G
        dq1, _, _ = _gpu_grads(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                               do[b:b + 1, h:h + 1], causal)
        assert torch.equal(dq1[0, 0].cpu(), dq[b, h].cpu()), (b, h)
