"""Seeded random shapes (fixed seeds, so every run checks the same cases) through the forward,
backward, variable-length and window/ALiBi paths against the fp64 oracle: odd query-head group
sizes, lengths on and off tile boundaries, both head dims and dtypes, causal and not.  Tolerances
as in the other parity tests."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import draw, draw_varlen, round_to
from gpu_util import device, f64, to_dev
from oracle import attention as A
from oracle import variants as VA
from oracle import varlen as VL

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.5e-2}
TOL_G = {"fp16": 5e-3, "bf16": 3e-2}
TOL_LSE = 1e-3


def _shape(i):
    r = np.random.default_rng(5000 + i)
    Hkv = int(r.integers(1, 4))
    G = int(r.integers(1, 5))
    N = int(r.choice([int(r.integers(1, 1300)), 64 * int(r.integers(1, 20)), 256 * int(r.integers(1, 5)) + 1]))
    return dict(B=int(r.integers(1, 3)), Hq=Hkv * G, Hkv=Hkv, N=N, d=int(r.choice([64, 128])),
                dtype=str(r.choice(["fp16", "bf16"])), causal=bool(r.integers(0, 2)))


@pytest.mark.parametrize("i", range(16))
def test_random_dense_fwd_bwd(i):
    s = _shape(i)
    print(f"[case] {s}", flush=True)
    _, q, k, v, do = draw(s["B"], s["Hq"], s["Hkv"], s["N"], s["d"], 6000 + i, with_grad=True)
    qc, kc, vc, doc = (round_to(x, s["dtype"]) for x in (q, k, v, do))
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (qc, kc, vc, doc))
    o, lse = eao.fwd(tq, tk, tv, causal=s["causal"])
    dq, dk, dv = eao.bwd(tq, tk, tv, o, tdo, lse, causal=s["causal"])
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(s["d"])
    ro, rl = A.forward(qc, kc, vc, s["causal"], scale)
    assert np.abs(f64(o) - ro).max() <= TOL_O[s["dtype"]]
    assert np.abs(f64(lse) - rl).max() <= TOL_LSE
    for got, ref in zip((dq, dk, dv), A.backward(qc, kc, vc, doc, s["causal"], scale)):
        assert np.abs(f64(got) - ref).max() <= TOL_G[s["dtype"]]


@pytest.mark.parametrize("i", range(8))
def test_random_varlen_fwd_bwd(i):
    r = np.random.default_rng(7000 + i)
    nseq = int(r.integers(1, 9))
    lens = [int(x) for x in r.integers(0, 600, size=nseq)]
    if sum(lens) == 0:
        lens[0] = 1
    Hkv = int(r.integers(1, 3))
    Hq = Hkv * int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    dtype = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    print(f"[case] lens={lens} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal}", flush=True)
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, d, 7100 + i)
    do = np.random.Generator(np.random.PCG64(7200 + i)).standard_normal(q.shape, dtype=np.float32)
    qc, kc, vc, doc = (round_to(x, dtype) for x in (q, k, v, do))
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (qc, kc, vc, doc))
    tcu = torch.from_numpy(cu).to(dev)
    ms = max(lens)
    o, lse = eao.fwd_varlen(tq, tk, tv, tcu, ms, causal=causal)
    dq, dk, dv = eao.bwd_varlen(tq, tk, tv, o, tdo, lse, tcu, ms, causal=causal)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    ro, rl = VL.forward(qc, kc, vc, cu, causal, scale)
    T = int(cu[-1])
    assert np.abs(f64(o)[:, :T] - ro[:, :T]).max() <= TOL_O[dtype]
    assert np.abs(f64(lse)[:, :T] - rl[:, :T]).max() <= TOL_LSE
    for got, ref in zip((dq, dk, dv), VL.backward(qc, kc, vc, doc, cu, causal, scale)):
        assert np.abs(f64(got) - ref).max() <= TOL_G[dtype]


@pytest.mark.parametrize("i", range(8))
def test_random_window_alibi_fwd_bwd(i):
    r = np.random.default_rng(8000 + i)
    Hkv = int(r.integers(1, 3))
    Hq = Hkv * int(r.integers(1, 4))
    N = int(r.integers(1, 900))
    d = int(r.choice([64, 128]))
    dtype = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    window = int(r.choice([0, int(r.integers(1, 400))]))
    alibi = bool(r.integers(0, 2)) or window == 0
    print(f"[case] N={N} Hq={Hq} Hkv={Hkv} d={d} {dtype} causal={causal} window={window} alibi={alibi}", flush=True)
    _, q, k, v, do = draw(1, Hq, Hkv, N, d, 8100 + i, with_grad=True)
    qc, kc, vc, doc = (round_to(x, dtype) for x in (q, k, v, do))
    slopes = (2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq)).astype(np.float32) if alibi else None
    dev = device()
    tq, tk, tv, tdo = (to_dev(x, dev) for x in (qc, kc, vc, doc))
    ts = None if slopes is None else torch.from_numpy(slopes).to(dev)
    o, lse = eao.fwd_ext(tq, tk, tv, causal=causal, window=window, alibi_slopes=ts)
    dq, dk, dv = eao.bwd_ext(tq, tk, tv, o, tdo, lse, causal=causal, window=window, alibi_slopes=ts)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    ro, rl = VA.forward(qc, kc, vc, causal, scale, window=window, slopes=slopes)
    assert np.abs(f64(o) - ro).max() <= TOL_O[dtype]
    assert np.abs(f64(lse) - rl).max() <= TOL_LSE
    for got, ref in zip((dq, dk, dv), VA.backward(qc, kc, vc, doc, causal, scale, window=window, slopes=slopes)):
        assert np.abs(f64(got) - ref).max() <= TOL_G[dtype]
