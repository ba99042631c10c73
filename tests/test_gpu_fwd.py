"""GPU parity of the forward kernels against the fp64 oracle (through the C ABI).

Tolerances: O max-abs error <= 2e-3 (fp16) / 1.5e-2 (bf16) on unit-normal inputs; LSE max-abs
<= 1e-3 (the statistics are fp32).  Every output is compared element by element, the large
workloads included (the oracle walks them in blocks of query rows).
"""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao
from attn_inputs import WORKLOADS, draw, round_to
from gpu_util import device, f64, sample_rows, to_dev
from oracle import attention as A

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 2e-3, "bf16": 1.5e-2}
TOL_LSE = 1e-3


def _inputs(B, Hq, Hkv, N, d, dtype, seed):
    _, q, k, v, _ = draw(B, Hq, Hkv, N, d, seed)
    return round_to(q, dtype), round_to(k, dtype), round_to(v, dtype)


def _run(q, k, v, causal, scale=None):
    dev = device()
    o, lse = eao.fwd(to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 127, 129, 200, 515])
def test_forward_small_full(dtype, d, causal, N):
    B, Hq, Hkv = 2, 3, 3
    q, k, v = _inputs(B, Hq, Hkv, N, d, dtype, seed=N * 7 + d + causal)
    o, lse = _run(q, k, v, causal)
    ro, rlse = A.forward(q, k, v, causal, 1.0 / np.sqrt(d))
    assert np.abs(f64(o) - ro).max() <= TOL_O[dtype]
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (4, 2), (8, 8), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_gqa_full(Hq, Hkv, causal):
    q, k, v = _inputs(2, Hq, Hkv, 300, 128, "bf16", seed=Hq * 10 + Hkv)
    o, lse = _run(q, k, v, causal)
    ro, rlse = A.forward(q, k, v, causal, 1.0 / np.sqrt(128))
    assert np.abs(f64(o) - ro).max() <= TOL_O["bf16"]
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE


def test_small_fp16_workload_full():
    w = WORKLOADS["small_fp16"]
    q, k, v = _inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, seed=1)
    o, lse = _run(q, k, v, w.causal)
    ro, rlse = A.forward(q, k, v, w.causal, w.scale)
    assert np.abs(f64(o) - ro).max() <= TOL_O["fp16"]
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE


def _full_check(w, seed, causal, row_block=1024):
    """Every O and LSE element of workload `w` against the oracle."""
    q, k, v = _inputs(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, seed=seed)
    o, lse = _run(q, k, v, causal)
    ro, rlse = A.forward(q, k, v, causal, w.scale, row_block=row_block)
    eo, el = np.abs(f64(o) - ro).max(), np.abs(f64(lse) - rlse).max()
    print(f"  {w.name} causal={causal}: O {eo:.3e}, LSE {el:.3e}", flush=True)
    assert eo <= TOL_O[w.dtype]
    assert el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_ablation_workload_full(causal):
    """B=8, H=16, N=2048, d=128, bf16: every output."""
    _full_check(WORKLOADS["ablation_bf16"], 2, causal)


@pytest.mark.timeout(900)
def test_long_workload_full():
    """B=1, H=16, N=16384, d=128, bf16, causal: every output."""
    _full_check(WORKLOADS["long_bf16"], 3, True)


@pytest.mark.timeout(900)
def test_gqa_workload_full():
    """B=4, Hq=32, Hkv=8, N=4096, d=128, bf16, causal: every output."""
    _full_check(WORKLOADS["gqa_bf16"], 4, True)


# ---------------------------------------------------------------- invariants on the device
@pytest.mark.parametrize("causal", [False, True])
def test_one_key_returns_v_exactly(causal):
    q, k, v = _inputs(2, 4, 2, 1, 128, "bf16", seed=5)
    o, lse = _run(q, k, v, causal)
    assert torch.equal(o.cpu(), v.repeat_interleave(2, dim=1))


def test_causal_row0_is_v0_exactly():
    q, k, v = _inputs(1, 2, 2, 333, 128, "bf16", seed=6)
    o, _ = _run(q, k, v, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_causal_future_keys_do_not_matter_bitwise():
    q, k, v = _inputs(1, 2, 2, 400, 128, "bf16", seed=7)
    o1, l1 = _run(q, k, v, True)
    i = 150
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i + 1:] = -k2[:, :, i + 1:] * 3
    v2[:, :, i + 1:] = v2[:, :, i + 1:] * 5
    o2, l2 = _run(q, k2, v2, True)
    assert torch.equal(o1[:, :, : i + 1], o2[:, :, : i + 1])
    assert torch.equal(l1[:, :, : i + 1], l2[:, :, : i + 1])


def test_uniform_scores_average_v():
    N = 300
    _, k, v = _inputs(1, 1, 1, N, 128, "bf16", seed=8)
    q = torch.zeros_like(k)
    o, lse = _run(q, k, v, False)
    want = f64(v).mean(axis=2, keepdims=True)
    assert np.abs(f64(o) - want).max() <= 2e-3
    assert np.abs(f64(lse) - np.log(N)).max() <= 1e-4


def test_forward_is_deterministic():
    q, k, v = _inputs(2, 4, 4, 700, 128, "bf16", seed=9)
    o1, l1 = _run(q, k, v, True)
    o2, l2 = _run(q, k, v, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_custom_scale():
    q, k, v = _inputs(1, 2, 2, 130, 64, "fp16", seed=10)
    o, lse = _run(q, k, v, False, scale=0.05)
    ro, rlse = A.forward(q, k, v, False, 0.05)
    assert np.abs(f64(o) - ro).max() <= TOL_O["fp16"]
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE


# ---------------------------------------------------------------- running-maximum growth
def _ramp_inputs(kind, N, d, dtype, seed):
    """Q rows and K rows along one direction u with key weights that ramp up ('up': the running
    maximum grows by far more than 2^8 from tile to tile, so the rescale of the accumulator runs
    on every tile), ramp down ('down': the first tile holds the maximum) or stay small but for one
    late key ('spike': one jump).  Scores reach about 100 (natural units).  'stairs' raises the
    level by about 6 log2 units per 64-key tile and 'plateau' once, after the first tile: a lane's
    32 keys of such a tile then sum to far more than 2^8 against the running maximum while the
    maximum itself grows by less than 2^8, so the d = 128 kernels rescale on the row-sum test
    alone (and recompute the tile's probabilities)."""
    g = np.random.Generator(np.random.PCG64(seed))
    u = g.standard_normal(d)
    u /= np.linalg.norm(u)
    t = np.arange(N) / max(N - 1, 1)
    step = 6.0 / (30.0 / np.sqrt(d) * np.log2(np.e))     # key weight of 6 log2 units of score
    alpha = {"up": 38.0 * t, "down": 38.0 * (1.0 - t), "spike": np.where(np.arange(N) == (7 * N) // 8, 38.0, 1.0),
             "stairs": step * (np.arange(N) // 64), "plateau": step * (np.arange(N) >= 64)}[kind]
    q = (30.0 * u)[None, :] + 0.3 * g.standard_normal((N, d))
    k = alpha[:, None] * u[None, :] + 0.3 * g.standard_normal((N, d))
    v = g.standard_normal((N, d))
    shape = (1, 1, N, d)
    return tuple(round_to(x.reshape(shape).astype(np.float32), dtype) for x in (q, k, v))


@pytest.mark.parametrize("kind", ["up", "down", "spike", "stairs", "plateau"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_running_maximum_growth(kind, dtype, causal):
    # O here is a sharp average of a few V rows (|O| up to max |V|, about 3.5, against ~0.05 for
    # unit-normal inputs), so the bar is the unit-normal one relative to max(1, max |O|)
    q, k, v = _ramp_inputs(kind, 515, 128, dtype, seed=11)
    o, lse = _run(q, k, v, causal)
    ro, rlse = A.forward(q, k, v, causal, 1.0 / np.sqrt(128))
    assert np.abs(f64(o) - ro).max() <= TOL_O[dtype] * max(1.0, np.abs(ro).max())
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE


# ---------------------------------------------------------------- block size chosen by grid size
# 256-row blocks (8 waves) when B*Hq*ceil(N/256) >= 512 and, for d = 128, the rows are not short
# (N > 2048, and N > 4096 when causal); else 128-row blocks (4 waves).  Below: 1*32*ceil(4200/256)
# = 544 blocks at d = 128 (N = 4200 = 16*256 + 104) and 2*64*ceil(1100/256) = 640 at d = 64, so
# the 8-wave path, over every output with a ragged tail; one head alone takes the 4-wave path,
# and each row's arithmetic is the same in both, so the two agree bit for bit.
@pytest.mark.parametrize("dtype,d,B,Hq,Hkv,N,heads", [("bf16", 128, 1, 32, 8, 4200, ((0, 0), (0, 17), (0, 31))),
                                                     ("fp16", 64, 2, 64, 16, 1100, ((0, 0), (1, 37), (1, 63)))])
@pytest.mark.parametrize("causal", [False, True])
def test_large_grid_full_and_block_size_invariance(dtype, d, B, Hq, Hkv, N, heads, causal):
    assert B * Hq * ((N + 255) // 256) >= 512
    assert not (d == 128 and (N <= 2048 or (causal and N <= 4096)))
    q, k, v = _inputs(B, Hq, Hkv, N, d, dtype, seed=20 + d + causal)
    o, lse = _run(q, k, v, causal)
    ro, rlse = A.forward(q, k, v, causal, 1.0 / np.sqrt(d))
    assert np.abs(f64(o) - ro).max() <= TOL_O[dtype]
    assert np.abs(f64(lse) - rlse).max() <= TOL_LSE
    G = Hq // Hkv
    for b, h in heads:
        g = h // G
        o1, l1 = _run(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], causal)
        assert torch.equal(o1[0, 0].cpu(), o[b, h].cpu()), (b, h)
        assert torch.equal(l1[0, 0].cpu(), lse[b, h].cpu()), (b, h)


@pytest.mark.parametrize("causal", [False, True])
def test_small_batch_heads_workload_sampled(causal):
    # B=1, H=16, N=2048, d=128: 128 blocks of 256 rows, so the 4-wave path with 256 blocks
    q, k, v = _inputs(1, 16, 16, 2048, 128, "bf16", seed=21 + causal)
    o, lse = _run(q, k, v, causal)
    rows = sample_rows(2048, seed=21)
    for h in (0, 7, 15):
        ro, rlse = A.forward_rows(q, k, v, causal, 1.0 / np.sqrt(128), 0, h, rows)
        assert np.abs(f64(o)[0, h, rows] - ro).max() <= TOL_O["bf16"], h
        assert np.abs(f64(lse)[0, h, rows] - rlse).max() <= TOL_LSE, h
