"""Plain fp64 attention for few query rows against a long key sequence, and the split/merge of
the keys that decoding uses.  TEST INFRASTRUCTURE.

Sources (page title + section):
  * "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning"
    (OpenReview discussion): the author response on decoding with long sequences (the key/value
    cache) and the review summary, in which the KV cache is split among thread blocks; the
    forward keeps one logsumexp per query row.
  * "FlashAttention (NeurIPS 2022)" study notes, "(Safe) Softmax" and "Online Softmax": a softmax
    over a set of keys can be assembled from the maxima and sums of disjoint parts.  With each
    part's normalised output O_s and logsumexp LSE_s, the whole is
        LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
    which is exact (the same identity the online softmax applies one block at a time).

Reading where the pages are silent (recorded in the design notes): with Nq < Nk query rows, the
queries are the last Nq positions of the sequence (bottom-right alignment): under causal masking
query i, at position Nk - Nq + i, sees keys j <= Nk - Nq + i.  With Nq = Nk this is the causal
mask of the square case.

The full result is the definition (attention.scores / attention.softmax_rows over all keys); the
split functions follow the method's steps: per split the plain definition restricted to the
split's keys, then the merge above.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["forward", "split_bounds", "split_partials", "merge"]


def _check(q, k, v):
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (B, d) != (Bk, dk) or v.shape != k.shape or Hkv < 1 or Hq % Hkv or Nq > Nk:
        raise ValueError(f"incompatible shapes q{q.shape} k{k.shape} v{v.shape}")
    return B, Hq, Hkv, Nq, Nk, d, Hq // Hkv


def forward(q, k, v, causal: bool, scale: float):
    """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] of q against k/v with Nk keys (bottom-right causal)."""
    q, k, v = A.as64(q), A.as64(k), A.as64(v)
    B, Hq, Hkv, Nq, Nk, d, G = _check(q, k, v)
    pos = np.arange(Nq) + (Nk - Nq)                     # positions of the query rows
    o = np.empty((B, Hq, Nq, d))
    lse = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            s = A.scores(q[b, h], k[b, h // G], scale, pos, causal)
            p, m, l = A.softmax_rows(s)
            o[b, h] = p @ v[b, h // G]
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def split_bounds(Nk: int, splits: int):
    """Contiguous key ranges [a, b) covering 0..Nk in `splits` nearly equal parts."""
    edges = np.linspace(0, Nk, splits + 1).round().astype(int)
    return [(int(edges[i]), int(edges[i + 1])) for i in range(splits)]


def split_partials(q, k, v, causal: bool, scale: float, bounds):
    """Per key range: (O_s [B,Hq,Nq,d], LSE_s [B,Hq,Nq]) over that range's keys only.  A row that
    sees none of the range's keys has O_s = 0 and LSE_s = -inf."""
    q, k, v = A.as64(q), A.as64(k), A.as64(v)
    B, Hq, Hkv, Nq, Nk, d, G = _check(q, k, v)
    pos = np.arange(Nq) + (Nk - Nq)
    out = []
    for a, e in bounds:
        o = np.zeros((B, Hq, Nq, d))
        lse = np.full((B, Hq, Nq), -np.inf)
        if e > a:
            keys = np.arange(a, e)
            for b in range(B):
                for h in range(Hq):
                    s = scale * (q[b, h] @ k[b, h // G, a:e].T)
                    if causal:
                        s = np.where(keys[None, :] > pos[:, None], -np.inf, s)
                    p, m, l = A.softmax_rows(s)
                    o[b, h] = p @ v[b, h // G, a:e]
                    with np.errstate(divide="ignore"):
                        lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
        out.append((o, lse))
    return out


def merge(partials):
    """Combine (O_s, LSE_s) of disjoint key sets: LSE = ln sum exp(LSE_s), O = sum exp(LSE_s - LSE) O_s."""
    lses = np.stack([p[1] for p in partials])           # [S, ...]
    mx = lses.max(axis=0)
    finite = np.isfinite(mx)
    mx_safe = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - mx_safe[None]), 0.0)
    wsum = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(wsum > 0, mx_safe + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
        o = sum(w[i][..., None] * partials[i][0] for i in range(len(partials)))
        o = np.where(wsum[..., None] > 0, o / np.where(wsum > 0, wsum, 1.0)[..., None], 0.0)
    return o, lse
