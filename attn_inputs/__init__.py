"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds no attention arithmetic: it only draws random numbers, rounds them to the
storage dtype a caller asks for, and names the workload shapes.  Both the CPU oracle and the
HIP path consume exactly what it returns, so neither side ever produces the other's inputs.

Recipe (applies to every workload):
  * generator: ``numpy.random.Generator(PCG64(seed))``;
  * draw order: Q, K, V, then dO (only when a backward is asked for), each with
    ``standard_normal(shape, dtype=float32)``;
  * rounding to fp16/bf16 is round-to-nearest-even through torch's dtype conversion;
  * decoding shapes (few query rows against a long key sequence): Q [B,Hq,Nq,d] then K, V
    [B,Hkv,Nk,d], same generator and order;
  * packed variable-length batches: the sequence lengths first (``varlen_lengths``: integers
    uniform in [lo, hi] from their own generator), then Q [Hq,T,d], K, V [Hkv,T,d] with T the sum
    of the lengths, same order as above;
  * fp8 extras (drawn after dO would be, from the same generator): for each of Q, K, V in that
    order, ``round(0.001 * numel)`` distinct flat indices chosen uniformly without replacement,
    whose entries are multiplied by 10 (outliers); then one sign vector of length d with entries
    +-1 (the random signs of the incoherent-processing transform);
  * tensors too large to draw on the host (``draw_on_device``): torch's generator on the device,
    seeded, ``randn`` in float32, then rounded like the rest; the oracle gets copies of the heads
    it checks.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "DECODE_WORKLOADS", "DecodeWorkload", "draw", "draw_decode", "draw_fp8",
           "draw_on_device", "draw_varlen", "varlen_lengths", "round_to", "DTYPES"]

DTYPES = ("fp16", "bf16")


@dataclass(frozen=True)
class Workload:
    """One attention problem: tensor shapes, storage dtype and mask."""

    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "fp16" | "bf16" | "fp8"
    causal: bool
    backward: bool

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        fields = dict(self.__dict__)
        fields.update(kw)
        return Workload(**fields)


# The five problems: a small fp16 forward, the B=8/H=16/N=2k ablation shape, the N=16k long
# sequence fwd+bwd, grouped-query attention with 4 query heads per K/V head, and the fp8 forward.
WORKLOADS = {
    "small_fp16": Workload("small_fp16", 1, 1, 1, 256, 64, "fp16", False, False),
    "ablation_bf16": Workload("ablation_bf16", 8, 16, 16, 2048, 128, "bf16", True, False),
    "long_bf16": Workload("long_bf16", 1, 16, 16, 16384, 128, "bf16", True, True),
    "gqa_bf16": Workload("gqa_bf16", 4, 32, 8, 4096, 128, "bf16", True, True),
    "fp8": Workload("fp8", 4, 16, 16, 4096, 128, "fp8", False, False),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """Decoding: Nq query rows per head against Nk keys (a K/V cache)."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# One new token per sequence (Nq = 1) for 8 sequences of 32k cached keys, 32 query heads sharing
# 8 K/V heads; and four tokens at once (speculative decoding) against 8k keys.
DECODE_WORKLOADS = {
    "decode_bf16": DecodeWorkload("decode_bf16", 8, 32, 8, 1, 32768, 128, "bf16", True),
    "decode4_bf16": DecodeWorkload("decode4_bf16", 4, 32, 8, 4, 8192, 128, "bf16", True),
}


def draw_decode(B, Hq, Hkv, Nq, Nk, d, seed):
    """Float32 Q [B,Hq,Nq,d], K, V [B,Hkv,Nk,d], N(0,1)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    q = gen.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    k = gen.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = gen.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    return q, k, v


def varlen_lengths(count, lo, hi, seed):
    """`count` sequence lengths, integers uniform in [lo, hi] (PCG64(seed))."""
    gen = np.random.Generator(np.random.PCG64(seed))
    return gen.integers(lo, hi + 1, size=count).astype(np.int64)


def draw_varlen(lengths, Hq, Hkv, d, seed):
    """Packed float32 Q [Hq,T,d], K, V [Hkv,T,d] (T = sum of lengths) and the int32 offsets
    cu_seqlens [len(lengths) + 1]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    gen = np.random.Generator(np.random.PCG64(seed))
    q = gen.standard_normal((Hq, T, d), dtype=np.float32)
    k = gen.standard_normal((Hkv, T, d), dtype=np.float32)
    v = gen.standard_normal((Hkv, T, d), dtype=np.float32)
    return q, k, v, cu


def round_to(x: np.ndarray, dtype: str):
    """Round float32 ``x`` to fp16/bf16 (RNE) and return a torch CPU tensor of that dtype."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "fp16":
        return t.to(torch.float16)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(B, Hq, Hkv, N, d, seed, with_grad=False):
    """Float32 Q [B,Hq,N,d], K, V [B,Hkv,N,d] and optionally dO [B,Hq,N,d], N(0,1)."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = g.standard_normal((B, Hkv, N, d), dtype=np.float32)
    v = g.standard_normal((B, Hkv, N, d), dtype=np.float32)
    do = g.standard_normal((B, Hq, N, d), dtype=np.float32) if with_grad else None
    return g, q, k, v, do


def draw_fp8(B, H, N, d, seed, outlier_frac=0.001, outlier_mult=10.0):
    """Float32 Q, K, V [B,H,N,d] with outliers, plus the +-1 sign vector (int8, length d)."""
    g, q, k, v, _ = draw(B, H, H, N, d, seed, with_grad=False)
    for t in (q, k, v):
        flat = t.reshape(-1)
        n_out = int(round(outlier_frac * flat.size))
        if n_out:
            idx = g.choice(flat.size, size=n_out, replace=False)
            flat[idx] *= np.float32(outlier_mult)
    signs = np.where(g.integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)
    return q, k, v, signs


def workload_inputs(w: Workload, seed: int):
    """Inputs for ``w`` at storage precision: torch CPU tensors (fp16/bf16) or float32 (fp8)."""
    if w.dtype == "fp8":
        q, k, v, signs = draw_fp8(w.B, w.Hq, w.N, w.d, seed)
        return {"q": q, "k": k, "v": v, "signs": signs}
    _, q, k, v, do = draw(w.B, w.Hq, w.Hkv, w.N, w.d, seed, with_grad=w.backward)
    out = {"q": round_to(q, w.dtype), "k": round_to(k, w.dtype), "v": round_to(v, w.dtype)}
    if do is not None:
        out["do"] = round_to(do, w.dtype)
    return out


def draw_on_device(shapes, dtype: str, seed: int, device):
    """One N(0,1) tensor per shape in ``shapes``, drawn in that order on ``device`` by torch's
    generator seeded with ``seed`` (float32, then rounded to fp16/bf16 as in round_to)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    out = []
    for shape in shapes:
        out.append(torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(tdt))
    return out
