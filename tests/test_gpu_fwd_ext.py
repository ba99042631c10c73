"""GPU parity of the forward with a sliding window and/or ALiBi (attn_fwd_ext) against the fp64
oracle.  Tolerances as for the plain forward: O max-abs <= 2e-3 (fp16) / 1.5e-2 (bf16), LSE
max-abs <= 1e-3."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, round_to
from gpu_util import device, f64, sample_rows, to_dev
from oracle import variants as VA

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def _inputs(B, Hq, Hkv, N, d, dtype, seed):
    _, q, k, v, _ = draw(B, Hq, Hkv, N, d, seed)
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def _slopes(Hq):
    return (2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq)).astype(np.float32)


def _run(q, k, v, causal, window, slopes):
    dev = device()
    ts = None if slopes is None else torch.from_numpy(slopes).to(dev)
    o, lse = eao.fwd_ext(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=causal, window=window,
                         alibi_slopes=ts)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


# fp16 at d = 128 runs the hand-scheduled fp16 tile step under the window masks (without ALiBi)
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("fp16", 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,window", [(1, 1), (63, 16), (200, 1), (200, 64), (515, 100), (515, 128), (300, 1000)])
@pytest.mark.parametrize("alibi", [False, True])
def test_fwd_ext_small_full(dtype, d, causal, N, window, alibi):
    B, Hq, Hkv = 2, 4, 2
    q, k, v = _inputs(B, Hq, Hkv, N, d, dtype, seed=N + window + d)
    sl = _slopes(Hq) if alibi else None
    o, lse = _run(q, k, v, causal, window, sl)
    ro, rlse = VA.forward(q, k, v, causal, 1.0 / np.sqrt(d), window=window, slopes=sl)
    # a small window with ALiBi concentrates a row on a few keys, so O reaches several times its
    # unit-normal size: the bar is the unit-normal one relative to max(1, max |O|), as the output's
    # own rounding and that of the probabilities scale with |O|
    assert np.abs(o - ro).max() <= TOL_O[dtype] * max(1.0, np.abs(ro).max())
    assert np.abs(lse - rlse).max() <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ext_alibi_only(causal):
    q, k, v = _inputs(1, 8, 8, 777, 128, "bf16", seed=12)
    sl = _slopes(8)
    o, lse = _run(q, k, v, causal, 0, sl)
    ro, rlse = VA.forward(q, k, v, causal, 1.0 / np.sqrt(128), slopes=sl)
    assert np.abs(o - ro).max() <= TOL_O["bf16"]
    assert np.abs(lse - rlse).max() <= TOL_LSE


def test_fwd_ext_plain_equals_fwd():
    q, k, v = _inputs(2, 4, 2, 333, 128, "bf16", seed=2)
    dev = device()
    o1, l1 = eao.fwd(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=True)
    o2, l2 = eao.fwd_ext(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=True)
    torch.cuda.synchronize()
    assert np.abs(f64(o1) - f64(o2)).max() <= 1e-2 and np.abs(f64(l1) - f64(l2)).max() <= 1e-5


@pytest.mark.parametrize("window,alibi", [(4096, True), (512, False)])
def test_fwd_ext_long_sampled_rows(window, alibi):
    # the long workload's shape (one batch, 16 heads, 16k keys) with a window, on sampled rows
    N, Hq = 16384, 16
    q, k, v = _inputs(1, Hq, Hq, N, 128, "bf16", seed=3)
    sl = _slopes(Hq) if alibi else None
    o, lse = _run(q, k, v, True, window, sl)
    rows = sample_rows(N, n_random=16, seed=window)
    for h in (0, 7, 15):
        ro, rl = VA.forward_rows(q, k, v, True, 1.0 / np.sqrt(128), window, sl, 0, h, rows)
        assert np.abs(o[0, h, rows] - ro).max() <= TOL_O["bf16"], h
        assert np.abs(lse[0, h, rows] - rl).max() <= TOL_LSE, h
