"""Plain fp64 attention with a local (sliding-window) mask and an ALiBi bias.  TEST INFRASTRUCTURE.

Source: "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning"
(OpenReview discussion, author responses): FA2 supports ALiBi, and local (sliding-window)
attention was used to train an open model.  The pages name both but define neither; the readings
below are recorded in the design notes:
  * window W > 0: key j is visible to query i only if i - j < W, and without the causal mask also
    j - i < W (a band of width 2W - 1 around the diagonal); with the causal mask, j <= i as well,
    so each row sees its last W positions;
  * ALiBi: score (i, j) of query head h is scale * q_i . k_j - slope_h * |i - j|, slopes given by
    the caller (one per query head).

The definition as written out: scores with the bias added, masked entries -inf, the safe softmax
of attention.softmax_rows, O = P V, LSE = m + ln l.  Backward ("FlashAttention (NeurIPS 2022)"
notes, "Backward - Recomputation"): the bias does not depend on Q or K, so the gradients of
L = <O, dO> are the chain rule of attention.block_grads applied to this P (masked entries have
P = 0 and contribute nothing).
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["forward", "forward_rows", "backward"]


def forward(q, k, v, causal: bool, scale: float, window: int = 0, slopes=None):
    """O [B,Hq,N,d] and LSE [B,Hq,N] with an optional window and ALiBi slopes (length Hq)."""
    q, k, v = A.as64(q), A.as64(k), A.as64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("incompatible shapes")
    G = Hq // Hkv
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    visible = np.ones((N, N), dtype=bool)
    if causal:
        visible &= j <= i
    if window > 0:
        visible &= (i - j) < window
        if not causal:
            visible &= (j - i) < window
    dist = np.abs(i - j).astype(np.float64)
    o = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // G].T)
            if slopes is not None:
                s = s - float(slopes[h]) * dist
            s = np.where(visible, s, -np.inf)
            p, m, l = A.softmax_rows(s)
            o[b, h] = p @ v[b, h // G]
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def forward_rows(q, k, v, causal: bool, scale: float, window: int, slopes, b: int, h: int, rows):
    """O and LSE of query head h of batch b for the given rows only (same definition as forward)."""
    q, k, v = A.as64(q), A.as64(k), A.as64(v)
    G = q.shape[1] // k.shape[1]
    N = k.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    i = rows[:, None]
    j = np.arange(N)[None, :]
    visible = np.ones((len(rows), N), dtype=bool)
    if causal:
        visible &= j <= i
    if window > 0:
        visible &= (i - j) < window
        if not causal:
            visible &= (j - i) < window
    s = scale * (q[b, h, rows] @ k[b, h // G].T)
    if slopes is not None:
        s = s - float(slopes[h]) * np.abs(i - j)
    s = np.where(visible, s, -np.inf)
    p, m, l = A.softmax_rows(s)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p @ v[b, h // G], lse


def _probs(q, k, causal, scale, window, slopes, b, h, G):
    N = k.shape[2]
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    visible = np.ones((N, N), dtype=bool)
    if causal:
        visible &= j <= i
    if window > 0:
        visible &= (i - j) < window
        if not causal:
            visible &= (j - i) < window
    s = scale * (q[b, h] @ k[b, h // G].T)
    if slopes is not None:
        s = s - float(slopes[h]) * np.abs(i - j)
    s = np.where(visible, s, -np.inf)
    p, _, _ = A.softmax_rows(s)
    return p


def backward(q, k, v, do, causal: bool, scale: float, window: int = 0, slopes=None):
    """dQ [B,Hq,N,d], dK, dV [B,Hkv,N,d] (fp64) of L = <O, dO> under the window / ALiBi of forward;
    dK and dV summed over the query heads that share each K/V head."""
    q, k, v, do = A.as64(q), A.as64(k), A.as64(v), A.as64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or do.shape != q.shape or Hq % Hkv:
        raise ValueError("incompatible shapes")
    G = Hq // Hkv
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(Hq):
            p = _probs(q, k, causal, scale, window, slopes, b, h, G)
            gq, gk, gv, _ = A.block_grads(p, do[b, h], q[b, h], k[b, h // G], v[b, h // G], scale)
            dq[b, h] = gq
            dk[b, h // G] += gk
            dv[b, h // G] += gv
    return dq, dk, dv
