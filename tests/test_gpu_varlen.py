"""GPU parity of the packed variable-length forward (attn_fwd_varlen) against the fp64 oracle.
Tolerances as for the plain forward: O max-abs <= 2e-3 (fp16) / 1.5e-2 (bf16), LSE <= 1e-3."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw_varlen, round_to, varlen_lengths
from gpu_util import device, f64, to_dev
from oracle import varlen as VL

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def _run(lens, Hq, Hkv, d, dtype, causal, seed, max_seqlen=None):
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, d, seed)
    q, k, v = round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)
    dev = device()
    ms = int(max(lens)) if max_seqlen is None else max_seqlen
    o, lse = eao.fwd_varlen(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), torch.from_numpy(cu).to(dev), ms,
                            causal=causal)
    torch.cuda.synchronize()
    return q, k, v, cu, f64(o), f64(lse)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("fp16", 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [[1], [300], [5, 0, 129, 1, 64], [128, 127, 255, 256, 2], [700, 33]])
def test_varlen_full(dtype, d, causal, lens):
    q, k, v, cu, o, lse = _run(lens, 4, 2, d, dtype, causal, seed=sum(lens) + d)
    ro, rlse = VL.forward(q, k, v, cu, causal, 1.0 / np.sqrt(d))
    T = int(cu[-1])
    assert np.abs(o[:, :T] - ro).max() <= TOL_O[dtype]
    assert np.abs(lse[:, :T] - rlse).max() <= TOL_LSE


def test_varlen_equals_separate_calls():
    lens = [200, 37, 512]
    q, k, v, cu, o, lse = _run(lens, 8, 8, 128, "bf16", True, seed=9)
    dev = device()
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        ob, lb = eao.fwd(to_dev(q[None, :, s0:s1], dev), to_dev(k[None, :, s0:s1], dev), to_dev(v[None, :, s0:s1], dev),
                         causal=True)
        torch.cuda.synchronize()
        assert np.array_equal(f64(ob)[0], o[:, s0:s1]) and np.array_equal(f64(lb)[0], lse[:, s0:s1])


def test_varlen_packed_workload_sampled_sequences():
    lens = varlen_lengths(16, 128, 8192, seed=3)
    q, k, v, cu, o, lse = _run(lens, 16, 16, 128, "bf16", True, seed=3)
    for b in (0, 7, 15):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ro, rlse = VL.forward(q[:2, s0:s1], k[:2, s0:s1], v[:2, s0:s1], np.array([0, s1 - s0]), True,
                              1.0 / np.sqrt(128))
        assert np.abs(o[:2, s0:s1] - ro).max() <= TOL_O["bf16"]
        assert np.abs(lse[:2, s0:s1] - rlse).max() <= TOL_LSE


def test_varlen_larger_max_seqlen_changes_nothing():
    # a grid sized for longer sequences only adds workgroups that return at once
    lens = [130, 64, 1, 250]
    a = _run(lens, 4, 4, 128, "bf16", True, seed=21)
    b = _run(lens, 4, 4, 128, "bf16", True, seed=21, max_seqlen=sum(lens))
    assert np.array_equal(a[4], b[4]) and np.array_equal(a[5], b[5])


def test_varlen_many_short_sequences():
    lens = list(varlen_lengths(64, 1, 40, seed=5))
    q, k, v, cu, o, lse = _run(lens, 2, 1, 64, "fp16", True, seed=5)
    ro, rlse = VL.forward(q, k, v, cu, True, 1.0 / np.sqrt(64))
    assert np.abs(o - ro).max() <= TOL_O["fp16"]
    assert np.abs(lse - rlse).max() <= TOL_LSE
