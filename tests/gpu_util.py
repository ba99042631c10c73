"""Helpers shared by the GPU parity tests (device tensors in, numpy float64 out)."""
import numpy as np
import pytest
import torch

import exact_attention_online_amd as eao


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    eao.load()          # raises if the HIP library is missing: there is no fallback
    return torch.device("cuda:0")


def to_dev(t, dev):
    return t.contiguous().to(dev)


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def sample_rows(N, n_random=48, seed=0, tile=128):
    """Edges of tiles and the tail plus random rows: indices into [0, N)."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, N - 1, N - 2, N // 2}
    for t in range(0, N, tile):
        rows.update({t, t - 1, t + 1, t + 31, t + 32, t + 63, t + 64})
    if len(rows) > 64:
        rows = set(sorted(rows)[:32]) | set(sorted(rows)[-32:])
    rows.update(rng.integers(0, N, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)


def half_step(ref, dtype):
    """Half the spacing of `dtype` (fp16/bf16) numbers at |ref|: the error that storing an exact
    value in that format can add by itself (round to nearest).  Zero for float32 outputs."""
    if dtype == "fp32":
        return np.zeros_like(np.asarray(ref, dtype=np.float64))
    mant = {"bf16": 7, "fp16": 10}[dtype]
    emin = {"bf16": -126, "fp16": -14}[dtype]
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mant - 1).astype(np.int64))


def excess(got, ref, tol, dtype):
    """max(|got - ref| - tol - half_step(ref)): <= 0 when every element is within the bar plus
    the rounding of the output format."""
    got = np.asarray(got, dtype=np.float64)
    return float((np.abs(got - ref) - tol - half_step(ref, dtype)).max())
