"""Plain fp64 attention over variable-length sequences packed without padding.  TEST
INFRASTRUCTURE.

Source: "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning"
(OpenReview discussion, author responses): variable sequence lengths are supported by
concatenating the sequences with no padding token, with an array giving the lengths.

Reading (recorded in the design notes): with the [B,H,N,d] layout of the rest of this oracle,
the B sequences are concatenated along the rows, q [Hq,T,d], k, v [Hkv,T,d]; sequence b occupies
rows cu[b] .. cu[b+1]-1 and attends only within itself (the causal mask applies per sequence).
Each sequence is the plain definition of attention.forward; its gradients are those of
attention.backward for that sequence alone ("FlashAttention (NeurIPS 2022)" notes, "Backward -
Recomputation"): L = <O, dO> summed over the sequences, and no gradient crosses from one sequence
to another.  Rows that belong to no sequence get zero gradients.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["forward", "backward"]


def forward(q, k, v, cu_seqlens, causal: bool, scale: float):
    """O [Hq,T,d] and LSE [Hq,T] of the packed sequences."""
    q, k, v = A.as64(q), A.as64(k), A.as64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    Hq, T, d = q.shape
    o = np.zeros((Hq, T, d))
    lse = np.zeros((Hq, T))
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 <= s0:
            continue
        ob, lb = A.forward(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], causal, scale)
        o[:, s0:s1] = ob[0]
        lse[:, s0:s1] = lb[0]
    return o, lse


def backward(q, k, v, do, cu_seqlens, causal: bool, scale: float):
    """dQ [Hq,T,d], dK, dV [Hkv,T,d] of the packed sequences (fp64); dK and dV summed over the
    query heads that share each K/V head, as in attention.backward."""
    q, k, v, do = A.as64(q), A.as64(k), A.as64(v), A.as64(do)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 <= s0:
            continue
        gq, gk, gv = A.backward(q[None, :, s0:s1], k[None, :, s0:s1], v[None, :, s0:s1], do[None, :, s0:s1],
                                causal, scale)
        dq[:, s0:s1] = gq[0]
        dk[:, s0:s1] = gk[0]
        dv[:, s0:s1] = gv[0]
    return dq, dk, dv
