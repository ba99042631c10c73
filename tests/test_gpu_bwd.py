"""GPU parity of the backward kernels against the fp64 oracle (through the C ABI).

Tolerances (max-abs over every compared element): dQ, dK, dV <= 5e-3 for fp16 and <= 3e-2 for
bf16 on unit-normal inputs.  The GPU backward consumes the GPU forward's O and LSE (the real
pipeline); one case feeds the oracle's O and LSE instead to isolate the backward kernels.
Every output is compared: small problems in one oracle call, the large workloads K/V head group
by K/V head group (every dK/dV row of the group and every dQ row of its query heads).

Gradient storage.  The bars are absolute.  A dK/dV sum over a group of query heads can exceed 8
in magnitude, where half a bfloat16 step (2^-5 = 0.03125) is itself more than 3e-2, so a bf16
result can miss the bar by its own rounding.  The contract checks therefore read the gradients in
float32 (grad_dtype=torch.float32: the kernels' fp32 accumulators written as they are) against
the plain bar, and the gradients stored in the input dtype against the bar plus half a step of
that dtype at the reference value (`gpu_util.excess`).
"""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import WORKLOADS, draw, round_to
from gpu_util import device, excess, f64, to_dev
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL = {"fp16": 5e-3, "bf16": 3e-2}


def _inputs(B, Hq, Hkv, N, d, dtype, seed):
    _, q, k, v, do = draw(B, Hq, Hkv, N, d, seed, with_grad=True)
    return [round_to(x, dtype) for x in (q, k, v, do)]


def _gpu_grads(q, k, v, do, causal, scale=None, o=None, lse=None, grad_dtype=None):
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    if o is None:
        o, lse = eao.fwd(tq, tk, tv, causal=causal, scale=scale)
    else:
        o, lse = to_dev(o, dev), to_dev(lse, dev)
    dq, dk, dv = eao.bwd(tq, tk, tv, o, tdo, lse, causal=causal, scale=scale, grad_dtype=grad_dtype)
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


def _every_group_check(w, seed, row_block):
    """Every output of workload `w`: float32 gradients against the bar, gradients stored in the
    input dtype against the bar plus half a step of that dtype; the oracle walks the K/V head
    groups one at a time."""
    q, k, v, do = _inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, seed=seed)
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (q, k, v, do))
    o, lse = eao.fwd(tq, tk, tv, causal=w.causal)
    g32 = eao.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, grad_dtype=torch.float32)
    g16 = eao.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal)
    torch.cuda.synchronize()
    for t in (*g32, *g16):
        assert torch.isfinite(t).all()
    q64, k64, v64, do64 = (f64(x) for x in (q, k, v, do))
    G = w.Hq // w.Hkv
    tol = TOL[w.dtype]
    worst = {}
    for b in range(w.B):
        for g in range(w.Hkv):
            rq, rk, rv, _ = A.backward_group(q64, k64, v64, do64, w.causal, w.scale, b, g, row_block=row_block)
            for name, idx, ref in (("dq", (b, slice(g * G, (g + 1) * G)), rq), ("dk", (b, g), rk), ("dv", (b, g), rv)):
                i = "dq dk dv".split().index(name)
                e32 = _err(g32[i][idx], ref)
                x16 = excess(f64(g16[i][idx]), ref, tol, w.dtype)
                worst[name] = max(worst.get(name, 0.0), e32)
                assert e32 <= tol, (name, b, g, e32)
                assert x16 <= 0.0, (name, b, g, x16)
        print(f"  batch {b}: worst float32 gradient errors so far {worst}", flush=True)


@pytest.mark.timeout(900)
def test_gqa_workload_every_group():
    """Grouped-query workload (B=4, Hq=32, Hkv=8, N=4096, d=128, bf16, causal): all 32 K/V groups."""
    _every_group_check(WORKLOADS["gqa_bf16"], 4, row_block=1024)


@pytest.mark.timeout(900)
def test_long_workload_every_head():
    """Long workload (B=1, H=16, N=16384, d=128, bf16, causal): all 16 heads."""
    _every_group_check(WORKLOADS["long_bf16"], 3, row_block=1024)


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
# The dQ kernel takes 256-row blocks (8 waves) when B*Hq*ceil(N/256) >= 512 and, at d = 128, the
# rows are not short (N > 2048, and N > 4096 when causal), else 128-row blocks (4 waves).  Below:
# 4*64*ceil(300/256) = 512 blocks, four query heads per K/V head, over every output with a ragged
# tail (300 = 256 + 44): the 8-wave path at d = 64, the 4-wave path at d = 128 (short rows; the
# next test covers its 8-wave path); one head alone takes the 4-wave path, and a row's
# arithmetic is the same in both, so its dQ agrees bit for bit.  Summed over four
# query heads dV reaches |11| here, where half a bf16 step is 2^-5 > 3e-2: float32 gradients are
# held to the bar, bf16 gradients to the bar plus their own rounding.
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_grid_full_and_block_size_invariance(dtype, d, causal):
    B, Hq, Hkv, N = 4, 64, 16, 300
    assert B * Hq * ((N + 255) // 256) >= 512
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, dtype, seed=90 + d + causal)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal, grad_dtype=torch.float32)
    dq16, dk16, dv16 = _gpu_grads(q, k, v, do, causal)
    rq, rk, rv = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(d))
    for got, got16, ref in ((dq, dq16, rq), (dk, dk16, rk), (dv, dv16, rv)):
        assert _err(got, ref) <= TOL[dtype]
        assert excess(f64(got16), ref, TOL[dtype], dtype) <= 0.0
        # the stored gradients are the float32 ones rounded to nearest
        assert torch.equal(got.to(got16.dtype), got16)
    G = Hq // Hkv
    for b, h in ((0, 0), (2, 37), (3, 63)):
        g = h // G
        dq1, _, _ = _gpu_grads(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                               do[b:b + 1, h:h + 1], causal)
        assert torch.equal(dq1[0, 0].cpu(), dq16[b, h].cpu()), (b, h)


# The 8-wave dQ path at d = 128: B=1, Hq=32, Hkv=8, N=4200 (1*32*17 = 544 blocks, rows past the
# short-row limits, ragged tail 4200 = 16*256 + 104).  dQ of three heads agrees bit for bit with
# one-head launches (4-wave path); the first K/V group (its four query heads) against the oracle.
@pytest.mark.parametrize("causal", [False, True])
def test_backward_dq_long_rows_block_size_invariance(causal):
    B, Hq, Hkv, N, d = 1, 32, 8, 4200, 128
    assert B * Hq * ((N + 255) // 256) >= 512 and N > 4096
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, "bf16", seed=95 + causal)
    dq, dk, dv = _gpu_grads(q, k, v, do, causal, grad_dtype=torch.float32)
    G = Hq // Hkv
    for h in (0, 17, 31):
        g = h // G
        dq1, _, _ = _gpu_grads(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], do[:, h:h + 1], causal,
                               grad_dtype=torch.float32)
        assert torch.equal(dq1[0, 0].cpu(), dq[0, h].cpu()), h
    rq, rk, rv = A.backward(q[:, 0:G], k[:, 0:1], v[:, 0:1], do[:, 0:G], causal, 1.0 / np.sqrt(d))
    assert _err(dq[:, 0:G], rq) <= TOL["bf16"]
    assert _err(dk[:, 0:1], rk) <= TOL["bf16"]
    assert _err(dv[:, 0:1], rv) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_float32_gradients_are_the_accumulators(dtype):
    """Both gradient dtypes come from the same accumulators: the stored ones are the float32
    ones rounded to nearest even, bit for bit, across the three phases as well."""
    B, Hq, Hkv, N, d = 2, 6, 2, 333, 128
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, dtype, seed=83)
    g32 = _gpu_grads(q, k, v, do, True, grad_dtype=torch.float32)
    g16 = _gpu_grads(q, k, v, do, True)
    refs = A.backward(q, k, v, do, True, 1.0 / np.sqrt(d))
    for a, b, r in zip(g32, g16, refs):
        assert a.dtype == torch.float32 and b.dtype == q.dtype
        assert torch.equal(a.to(b.dtype), b)
        assert _err(a, r) <= TOL[dtype]


# ---------------------------------------------------------------- split dK/dV phase (small grouped grids)
# With few K/V heads and keys (B * Hkv * ceil(N / 128) < 256) the dK/dV phase cuts each key block's
# (query head, query tile) steps into ranges, keeps each range's share in fp32 and adds the shares
# in a fixed order.  B=1, Hq=16, Hkv=2, N=2048: 32 key blocks, 16 ranges each.
@pytest.mark.parametrize("causal", [False, True])
def test_split_dkdv_small_grouped_grid_full(causal):
    B, Hq, Hkv, N, d = 1, 16, 2, 2048, 128
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, "bf16", seed=120 + causal)
    g32 = _gpu_grads(q, k, v, do, causal, grad_dtype=torch.float32)
    g16 = _gpu_grads(q, k, v, do, causal)
    refs = A.backward(q, k, v, do, causal, 1.0 / np.sqrt(d))
    for a, b, r in zip(g32, g16, refs):
        assert _err(a, r) <= TOL["bf16"]
        assert torch.equal(a.to(torch.bfloat16), b)
    # deterministic: the shares are added in a fixed order
    again = _gpu_grads(q, k, v, do, causal, grad_dtype=torch.float32)
    for a, b in zip(g32, again):
        assert torch.equal(a, b)


@pytest.mark.parametrize("Hq,Hkv,N", [(8, 1, 129), (6, 2, 1), (32, 4, 700), (12, 3, 64)])
def test_split_dkdv_edge_shapes(Hq, Hkv, N):
    """Ranges that start inside a head's tiles, single-tile heads, ragged tails, one key."""
    q, k, v, do = _inputs(1, Hq, Hkv, N, 128, "bf16", seed=130 + N)
    dq, dk, dv = _gpu_grads(q, k, v, do, True, grad_dtype=torch.float32)
    rq, rk, rv = A.backward(q, k, v, do, True, 1.0 / np.sqrt(128))
    assert _err(dq, rq) <= TOL["bf16"]
    assert _err(dk, rk) <= TOL["bf16"]
    assert _err(dv, rv) <= TOL["bf16"]
