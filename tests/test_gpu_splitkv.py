"""GPU parity of the split-KV (decoding) forward against the fp64 oracle, through the C ABI.

Tolerances as for the main forward: O max-abs <= 2e-3 (fp16) / 1.5e-2 (bf16), LSE max-abs
<= 1e-3.  Small problems are compared over every output, including more than 32 query rows per
K/V head (several 32-row groups); the decoding workloads (8 x 32 heads against 32k keys; 4 query
rows x 4 x 32 heads against 8k keys) on a sample of heads that the oracle computes head by head.
"""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import DECODE_WORKLOADS, draw_decode, round_to
from gpu_util import device, f64, to_dev
from oracle import decode as DC

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    q, k, v = draw_decode(B, Hq, Hkv, Nq, Nk, d, seed)
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def _run(q, k, v, causal, splits=0):
    dev = device()
    o, lse = eao.fwd_splitkv(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, dtype, causal, splits
    (1, 1, 1, 1, 1, 128, "bf16", False, 0),
    (1, 4, 1, 1, 1000, 128, "bf16", True, 0),
    (2, 8, 2, 4, 777, 128, "bf16", True, 3),
    (1, 32, 8, 1, 4097, 128, "bf16", True, 0),
    (2, 4, 4, 8, 300, 64, "fp16", True, 5),
    (1, 2, 1, 16, 129, 64, "bf16", False, 1),
    (1, 8, 1, 4, 2048, 128, "fp16", True, 64),
    (1, 2, 2, 20, 20, 128, "bf16", True, 2),
    (3, 6, 3, 3, 255, 128, "fp16", False, 2),
    (1, 16, 2, 4, 128, 64, "fp16", True, 0),
    # more than 32 rows per K/V head: several groups of 32 rows, the last one ragged
    (1, 32, 4, 8, 1500, 128, "bf16", True, 0),
    (2, 16, 1, 5, 700, 128, "bf16", True, 3),
    (1, 8, 8, 33, 1000, 64, "fp16", False, 2),
    (1, 40, 1, 1, 4096, 128, "bf16", False, 0),
    (1, 2, 1, 100, 100, 128, "fp16", True, 1),
    # more than 64 splits: the merge takes the logsumexps in chunks of 64 lanes, the last ragged
    (1, 8, 2, 2, 16700, 128, "bf16", True, 131),
    (1, 4, 1, 3, 9000, 64, "fp16", False, 71),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal,splits", CASES)
def test_splitkv_small_full(B, Hq, Hkv, Nq, Nk, d, dtype, causal, splits):
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed=Nk + 13 * Nq + d)
    o, lse = _run(q, k, v, causal, splits)
    ro, rlse = DC.forward(q, k, v, causal, 1.0 / np.sqrt(d))
    assert np.abs(o - ro).max() <= TOL_O[dtype]
    assert np.abs(lse - rlse).max() <= TOL_LSE


@pytest.mark.parametrize("splits", [1, 2, 5, 17, 0])
def test_splitkv_any_split_count(splits):
    q, k, v = _inputs(2, 8, 2, 2, 2100, 128, "bf16", seed=31)
    o, lse = _run(q, k, v, True, splits)
    ro, rlse = DC.forward(q, k, v, True, 1.0 / np.sqrt(128))
    assert np.abs(o - ro).max() <= TOL_O["bf16"]
    assert np.abs(lse - rlse).max() <= TOL_LSE


def test_square_case_matches_the_main_forward():
    # Nq = Nk: the bottom-right alignment is the ordinary causal mask
    q, k, v = _inputs(1, 4, 2, 8, 8, 128, "fp16", seed=5)
    o, lse = _run(q, k, v, True, 2)
    dev = device()
    o2, lse2 = eao.fwd(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=True)
    torch.cuda.synchronize()
    assert np.abs(o - f64(o2)).max() <= 2 * TOL_O["fp16"]
    assert np.abs(lse - f64(lse2)).max() <= TOL_LSE


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workloads_sampled_heads(name):
    w = DECODE_WORKLOADS[name]
    q, k, v = _inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, seed=7)
    o, lse = _run(q, k, v, w.causal)
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(3)
    for b, h in {(0, 0), (w.B - 1, w.Hq - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(4)}:
        g = h // G
        ro, rlse = DC.forward(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], w.causal, w.scale)
        assert np.abs(o[b, h] - ro[0, 0]).max() <= TOL_O[w.dtype], (b, h)
        assert np.abs(lse[b, h] - rlse[0, 0]).max() <= TOL_LSE, (b, h)


def test_row_groups_match_one_group_per_call():
    # 64 rows per K/V head (two groups of 32): each query head's result is bit for bit that of a
    # call on the heads of its 32-row group alone (a row's arithmetic does not depend on the
    # other rows of the launch)
    q, k, v = _inputs(1, 16, 2, 8, 1111, 128, "bf16", seed=17)
    o, lse = _run(q, k, v, True, 2)
    for g in range(2):
        for part in range(2):
            hs = slice(8 * g + 4 * part, 8 * g + 4 * part + 4)
            o1, l1 = _run(q[:, hs], k[:, g:g + 1], v[:, g:g + 1], True, 2)
            assert np.array_equal(o1, o[:, hs]) and np.array_equal(l1, lse[:, hs]), (g, part)


def test_workspace_contents_do_not_matter():
    q, k, v = _inputs(1, 8, 2, 2, 999, 128, "bf16", seed=9)
    dev = device()
    tq, tk, tv = (to_dev(x, dev) for x in (q, k, v))
    n = eao.splitkv_workspace_size(1, 8, 2, 2, 999, 128, 3)
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device=dev)
    a = eao.fwd_splitkv(tq, tk, tv, causal=True, num_splits=3, workspace=ws)
    b = eao.fwd_splitkv(tq, tk, tv, causal=True, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_one_long_sequence_sampled_heads():
    # one 131072-key sequence (automatic plan: 64 splits of 2048 keys per K/V head), a sample of
    # heads against the oracle
    B, Hq, Hkv, Nq, Nk, d = 1, 32, 8, 1, 131072, 128
    q, k, v = _inputs(B, Hq, Hkv, Nq, Nk, d, "bf16", seed=23)
    o, lse = _run(q, k, v, True)
    G = Hq // Hkv
    for h in (0, 13, 31):
        g = h // G
        ro, rlse = DC.forward(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], True, 1.0 / np.sqrt(d))
        assert np.abs(o[0, h] - ro[0, 0]).max() <= TOL_O["bf16"], h
        assert np.abs(lse[0, h] - rlse[0, 0]).max() <= TOL_LSE, h
