"""GPU parity of the fp8 path: the prep kernel (bit-exact) and the fp8 forward.

Three layers, following the reading of block quantisation + incoherent processing:
  1. prep: e4m3 codes and per-block scales equal the CPU quantiser's bit for bit (both take the
     rounding decisions in float32, the butterfly in the same stage order);
  2. kernel arithmetic: the fp8 forward against fp64 attention on the dequantised inputs, within
     a per-element bound derived from the only lossy step inside the kernel -- probabilities
     rounded to e4m3 -- plus the bf16 rounding of O.  The kernel converts p = P~ * 2^7 (P~ <= 2
     against a row maximum that is kept until a score passes it by more than 1 in log2 units):
     relative error <= 2^-4 in the normal range and absolute <= 2^-10 in p below it (half the
     e4m3 subnormal step), i.e. e_j <= max(2^-4 P~_j, 2^-17); rescaling by the growth of the
     maximum only shrinks both, and the V block scales are applied in fp32 to the accumulator.
     The row sum l is taken over the same rounded values (an MFMA against ones), so the kernel
     returns sum_j p^_j V_j / sum_j p^_j, whose distance from the exact O is
     |sum_j eps_j (V_j - O)| / (l + sum eps) <= (sum_j e_j |V_j| + |O| sum_j e_j) / (l - sum_j e_j),
     and its LSE is off by at most -ln(1 - sum_j e_j / l);
  3. the contract: O against the fp64 oracle on the unquantised inputs, RMSE <= 3e-2 over all
     elements, and (because that bar alone would pass an all-zero output on these inputs)
     relative RMSE <= 0.2.
"""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import WORKLOADS, draw_fp8
from gpu_util import device, f64
from oracle import attention as A
from oracle import fp8 as F

pytestmark = pytest.mark.gpu


def _prep_gpu(x, signs, pow2=False):
    dev = device()
    tx = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ts = None if signs is None else torch.from_numpy(signs).to(dev)
    codes, desc = eao.fp8_prep(tx, ts, pow2_scale=pow2)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), desc.cpu().numpy()


def _prep_ref(x, signs, pow2=False):
    y = F.incoherent_f32(x, signs) if signs is not None else np.asarray(x, np.float32)
    return F.block_quantize(y, pow2=pow2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 100, 128, 300, 1024])
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("pow2", [False, True])
def test_prep_bit_exact(d, N, hadamard, pow2):
    q, k, v, signs = draw_fp8(2, 3, N, d, seed=N + d)
    x = q if hadamard else v
    s = signs if hadamard else None
    codes, desc = _prep_gpu(x, s, pow2)
    rc, rd = _prep_ref(x, s, pow2)
    assert np.array_equal(desc, rd)
    assert np.array_equal(codes, rc), f"{(codes != rc).sum()} codes differ"


def test_prep_special_values():
    x = np.zeros((1, 1, 256, 128), np.float32)          # block 0 all zero -> scale 1, codes 0
    x[0, 0, 128:] = np.random.default_rng(0).standard_normal((128, 128)).astype(np.float32) * 1e-3
    x[0, 0, 200, 5] = -7.5                               # the block's amax lands on code -448
    codes, desc = _prep_gpu(x, None)
    rc, rd = _prep_ref(x, None)
    assert np.array_equal(codes, rc) and np.array_equal(desc, rd)
    assert desc[0, 0, 0] == 1.0 and np.all(codes[0, 0, :128] == 0)
    assert codes[0, 0, 200, 5] == 0xFE


def _fp8_pipeline(q, k, v, signs, causal, vpow2=True):
    """attn_fp8_prep (Hadamard on Q and K; V block scales powers of two unless vpow2 is False,
    which takes the kernel's accumulator-rescaling path) then attn_fwd in fp8."""
    dev = device()
    q8, qs = eao.fp8_prep(torch.from_numpy(q).to(dev), torch.from_numpy(signs).to(dev))
    k8, ks = eao.fp8_prep(torch.from_numpy(k).to(dev), torch.from_numpy(signs).to(dev))
    v8, vs = eao.fp8_prep(torch.from_numpy(v).to(dev), None, pow2_scale=vpow2)
    o, lse = eao.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=causal, scale=1.0 / np.sqrt(q.shape[-1]))
    torch.cuda.synchronize()
    return (q8.cpu().numpy(), qs.cpu().numpy(), k8.cpu().numpy(), ks.cpu().numpy(), v8.cpu().numpy(),
            vs.cpu().numpy(), f64(o), f64(lse))


def _kernel_bound(qd, kd, vd, causal, scale):
    """fp64 O and LSE on dequantised inputs, and the per-element bound of the fp8 kernel."""
    o, lse = A.forward(qd, kd, vd, causal, scale)
    G = qd.shape[1] // kd.shape[1]
    bound = np.empty_like(o)
    lse_bound = np.empty_like(lse)
    N = qd.shape[2]
    for b in range(qd.shape[0]):
        for h in range(qd.shape[1]):
            s = A.scores(qd[b, h], kd[b, h // G], scale, np.arange(N), causal)
            p, m, l = A.softmax_rows(s)
            pt = p * l[:, None]                                 # unnormalised P~ in [0, 1]
            perr = np.maximum(pt * 2.0 ** -4, 2.0 ** -17)       # e4m3 rounding of p (see above)
            if causal:
                perr = np.where(np.triu(np.ones((N, N), bool), 1), 0.0, perr)
            esum = perr.sum(axis=1)
            assert np.all(esum < 0.5 * l)
            bound[b, h] = (perr @ np.abs(vd[b, h // G]) + esum[:, None] * np.abs(o[b, h])) / (l - esum)[:, None]
            lse_bound[b, h] = -np.log1p(-esum / l)
    bound += 2.0 ** -8 * np.abs(o) + 1e-4                        # bf16 output rounding, fp32 sums
    lse_bound += 1e-5                                            # fp32 statistics
    return o, lse, bound, lse_bound


@pytest.mark.parametrize("N,causal,vpow2", [(64, False, True), (200, False, True), (333, True, True),
                                            (1000, False, True), (1000, True, True), (1000, False, False),
                                            (777, True, False)])
def test_fp8_forward_kernel_arithmetic(N, causal, vpow2):
    q, k, v, signs = draw_fp8(1, 2, N, 128, seed=900 + N)
    q8, qs, k8, ks, v8, vs, o, lse = _fp8_pipeline(q, k, v, signs, causal, vpow2)
    qd, kd, vd = F.dequantize(q8, qs), F.dequantize(k8, ks), F.dequantize(v8, vs)
    ro, rlse, bound, lse_bound = _kernel_bound(qd, kd, vd, causal, 1.0 / np.sqrt(128))
    err = np.abs(o - ro)
    assert np.all(err <= bound), f"worst excess {(err - bound).max():.3e}"
    lerr = np.abs(lse - rlse)
    print(f"  N={N} causal={causal}: O error / bound max {(err / bound).max():.3f}, LSE error max {lerr.max():.2e} "
          f"(bound max {lse_bound.max():.2e})", flush=True)
    assert np.all(lerr <= lse_bound), f"worst LSE excess {(lerr - lse_bound).max():.3e}"


def test_fp8_workload_contract():
    w = WORKLOADS["fp8"]
    q, k, v, signs = draw_fp8(w.B, w.Hq, w.N, w.d, seed=5)
    *_, o, lse = _fp8_pipeline(q, k, v, signs, w.causal)
    ro, rlse = A.forward(q, k, v, w.causal, w.scale, row_block=2048)   # unquantised inputs, fp64
    rmse = float(np.sqrt(np.mean((o - ro) ** 2)))
    rms_ref = float(np.sqrt(np.mean(ro ** 2)))
    lerr = np.abs(lse - rlse)
    print(f"  fp8 workload: RMSE {rmse:.3e}, RMS(ref) {rms_ref:.3e}, relative {rmse / rms_ref:.3f}, "
          f"max-abs {np.abs(o - ro).max():.3e}; LSE abs error mean {lerr.mean():.3e} max {lerr.max():.3e}",
          flush=True)
    assert rmse <= 3e-2
    assert rmse / rms_ref <= 0.2
    # the LSE against unquantised inputs carries the input quantisation error (no stated bar);
    # the kernel's own LSE arithmetic is bounded in test_fp8_forward_kernel_arithmetic
    assert np.isfinite(lse).all()


def test_fp8_error_ratio_study():
    """The FlashAttention-3 abstract reports lower numerical error for its fp8 attention (block
    quantisation + incoherent processing) than for a baseline fp8 attention.  Reading of the
    baseline: one scale per tensor, no Hadamard transform.  All four combinations run through the
    same fp8 kernel on the fp8 workload's inputs (0.1% outliers x 10); RMSE of O against the fp64
    definition on the unquantised inputs, on 8 heads.  The measured ratios are printed; the
    assertion only requires that each of the two techniques reduces the error."""
    w = WORKLOADS["fp8"]
    q, k, v, signs = draw_fp8(w.B, w.Hq, w.N, w.d, seed=5)
    dev = device()
    heads = [(0, 0), (0, 5), (1, 10), (1, 15), (2, 3), (2, 8), (3, 12), (3, 1)]
    ref = {}
    for b, h in heads:
        ro, _ = A.forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], w.causal, w.scale,
                          row_block=2048)
        ref[(b, h)] = ro[0, 0]

    def run(quant, hadamard, vquant=None):
        qq = F.incoherent_f32(q, signs) if hadamard else q
        kk = F.incoherent_f32(k, signs) if hadamard else k
        parts = [quant(qq), quant(kk), (vquant or quant)(v)]
        t = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for c_s in parts for a in c_s]
        o, _ = eao.fwd_fp8(t[0], t[2], t[4], t[1], t[3], t[5], causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        o = f64(o)
        err = np.concatenate([(o[b, h] - ref[(b, h)]).ravel() for b, h in heads])
        return float(np.sqrt(np.mean(err ** 2)))

    r_tensor = run(F.tensor_quantize, False)      # baseline
    r_tensor_had = run(F.tensor_quantize, True)
    r_block = run(F.block_quantize, False)
    r_block_had = run(F.block_quantize, True)
    # what attn_fp8_prep + attn_fwd compute: V with power-of-two block scales
    r_ours = run(F.block_quantize, True, lambda x: F.block_quantize(x, pow2=True))
    # the block-quantised, transformed inputs are exactly what the prep kernel produces
    _, _, _, _, _, _, o_gpu, _ = _fp8_pipeline(q, k, v, signs, w.causal)
    err = np.concatenate([(o_gpu[b, h] - ref[(b, h)]).ravel() for b, h in heads])
    assert abs(float(np.sqrt(np.mean(err ** 2))) - r_ours) <= 1e-6
    print(f"  fp8 error study (RMSE of O, 8 heads): per-tensor {r_tensor:.4e}, per-tensor + Hadamard "
          f"{r_tensor_had:.4e}, block {r_block:.4e}, block + Hadamard {r_block_had:.4e}, block + Hadamard "
          f"with power-of-two V scales (ours) {r_ours:.4e}; baseline / ours = {r_tensor / r_ours:.2f}", flush=True)
    assert r_block < r_tensor and r_ours < r_block


def _ramp_inputs(N, kind, seed):
    """Q, K whose scores grow along the keys by far more than the kernel's offset range: 'ramp' --
    every query is 10 e_0 and key j is 60 (j / N) e_0, so score (i, j) = 600 j / N / sqrt(d),
    about 76 log2 units from the first key to the last; 'jump' -- unit-normal scores with one key
    per 128 (after the first block) lifted by 90 log2 units over its neighbours.  V is the fp8
    workload's; the Hadamard signs are the draw's."""
    _, _, v, signs = draw_fp8(1, 2, N, 128, seed=seed)
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 2, N, 128), np.float32)
    k = np.zeros((1, 2, N, 128), np.float32)
    if kind == "ramp":
        q[..., 0] = 10.0
        k[..., 0] = (60.0 * np.arange(N) / N).astype(np.float32)
    else:
        q[:] = rng.standard_normal(q.shape).astype(np.float32)
        k[:] = rng.standard_normal(k.shape).astype(np.float32)
        lift = 90.0 / np.log2(np.e) * np.sqrt(128.0)        # 90 log2 units of score
        for j in range(192, N, 128):
            k[0, :, j] += lift * q[0, :, min(j, N - 1)] / np.maximum(
                np.sum(q[0, :, min(j, N - 1)] ** 2, axis=-1, keepdims=True), 1e-3)
    return q, k, v, signs


@pytest.mark.parametrize("kind", ["ramp", "jump"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_large_maximum_growth(kind, causal):
    """Rows whose maximum grows by more than 64 log2 units: the kernel's integer offset passes
    its limit and the row is rebased (accumulator and row sum times 2^-k), on top of the offsets
    applied through the MFMA scale operand.  The same per-element bound as the arithmetic test."""
    N = 1000
    q, k, v, signs = _ramp_inputs(N, kind, seed=1700 + N)
    q8, qs, k8, ks, v8, vs, o, lse = _fp8_pipeline(q, k, v, signs, causal)
    qd, kd, vd = F.dequantize(q8, qs), F.dequantize(k8, ks), F.dequantize(v8, vs)
    ro, rlse, bound, lse_bound = _kernel_bound(qd, kd, vd, causal, 1.0 / np.sqrt(128))
    s_c = (qd[0, 0] @ kd[0, 0].T) / np.sqrt(128) * np.log2(np.e)
    growth = (s_c.max(axis=1) - s_c[:, :64].max(axis=1)).max()
    assert growth > 64, f"the inputs grow the row maximum by only {growth:.1f} log2 units"
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    err = np.abs(o - ro)
    assert np.all(err <= bound), f"worst excess {(err - bound).max():.3e}"
    lerr = np.abs(lse - rlse)
    print(f"  {kind} causal={causal}: maximum growth {growth:.1f} log2 units, O error / bound max "
          f"{(err / bound).max():.3f}, LSE error max {lerr.max():.2e}", flush=True)
    assert np.all(lerr <= lse_bound), f"worst LSE excess {(lerr - lse_bound).max():.3e}"
