"""Tiled one-pass (online-softmax) attention forward in float64 -- a model of the algorithm.

TEST INFRASTRUCTURE.  It is checked against the plain definition in ``attention.py`` (they must
agree to rounding), which pins the reading of the recurrence, of causal block skipping and of
tail tiles.  GPU results are never compared against this model, only against the definition.

Sources (page title + section):
  * "FlashAttention (NeurIPS 2022)" notes, "Online Softmax": a running maximum m and running
    denominator d' are updated in one sweep, and the final d' equals the softmax denominator;
    "FlashAttention": the same idea carries the output accumulator o' along, so one loop gives
    O; the tiled form splits queries into B_r-row blocks and keys/values into B_c-row blocks and
    does not tile the head dimension.
  * "FlashAttention-2 ... (OpenReview discussion)", author responses: keep the accumulator
    unnormalised and divide by the denominator once at the end; save the logsumexp; blocks that
    lie wholly after the query block are skipped and the mask is applied to the diagonal block
    only.
"""
from __future__ import annotations

import numpy as np

from .attention import as64

__all__ = ["forward_tiled"]


def forward_tiled(q, k, v, causal: bool, scale: float, block_r: int, block_c: int):
    """Returns (O, LSE, visited) where visited counts the (query block, key block) pairs done."""
    q, k, v = as64(q), as64(k), as64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    visited = 0
    for b in range(B):
        for h in range(Hq):
            kg, vg = k[b, h // G], v[b, h // G]
            for r0 in range(0, N, block_r):
                rows = np.arange(r0, min(N, r0 + block_r))
                qi = q[b, h, rows]
                m = np.full(len(rows), -np.inf)   # running max
                l = np.zeros(len(rows))           # running denominator d'
                acc = np.zeros((len(rows), d))    # unnormalised o'
                last_key = rows[-1] if causal else N - 1
                for c0 in range(0, last_key + 1, block_c):   # key blocks after the query block are skipped
                    keys = np.arange(c0, min(N, c0 + block_c))
                    visited += 1
                    s = scale * (qi @ kg[keys].T)
                    if causal and keys[-1] > rows[0]:           # only blocks that cross the diagonal are masked
                        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m, s.max(axis=1))
                    alpha = np.exp(m - m_new)                     # exp(-inf) = 0 on the first block
                    pt = np.exp(s - m_new[:, None])
                    l = alpha * l + pt.sum(axis=1)
                    acc = alpha[:, None] * acc + pt @ vg[keys]
                    m = m_new
                o[b, h, rows] = acc / l[:, None]                  # one division at the end
                lse[b, h, rows] = m + np.log(l)
    return o, lse, visited
