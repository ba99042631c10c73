"""Plain fp64 attention over variable-length sequences packed without padding.  TEST
INFRASTRUCTURE.

Source: "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning"
(OpenReview discussion, author responses): variable sequence lengths are supported by
concatenating the sequences with no padding token, with an array giving the lengths.

Reading (recorded in the design notes): with the [B,H,N,d] layout of the rest of this oracle,
the B sequences are concatenated along the rows, q [Hq,T,d], k, v [Hkv,T,d]; sequence b occupies
rows cu[b] .. cu[b+1]-1 and attends only within itself (the causal mask applies per sequence).
Each sequence is the plain definition of attention.forward.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["forward"]


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
