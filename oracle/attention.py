"""Plain fp64 attention forward and backward -- the definition, written out.  TEST INFRASTRUCTURE.

Sources (page title + section):
  * "FlashAttention (NeurIPS 2022)" study notes, "From Online Softmax to FlashAttention": the
    attention result is X = Q K^T, A = softmax(X), O = A V; section "(Safe) Softmax": the softmax
    of a row subtracts the row maximum, exponentiates and divides by the row sum.
  * "FlashAttention-2 ... (OpenReview discussion)", author responses: the method is exact (no
    approximation), the forward saves one logsumexp per query row, the backward is a separate
    pass, dV = P^T dO where dO is the gradient of the loss with respect to O; causal masking
    removes key blocks that lie after the query ("they don't contribute to the outputs").
  * Same discussion, review 2 / response: grouped-query attention, where several query heads
    share one K/V head; dK and dV of a shared head collect the contributions of every query head
    in its group.

Readings where the pages are silent (each also recorded in the design notes):
  * layout [B, H, N, d]; query head h uses K/V head h // (Hq // Hkv);
  * softmax scale is a caller parameter (the workloads use 1/sqrt(d));
  * causal: key j is visible to query i iff j <= i (query and key lengths are equal);
  * LSE is the natural log, LSE_i = m_i + ln(l_i); a fully masked row would give O = 0 and
    LSE = -inf (not reachable with equal lengths);
  * the remaining gradient relations are the chain rule through O = P V and P = softmax(S):
    dP = dO V^T, dS = P * (dP - D) with D_i = sum_j P_ij dP_ij, dQ = scale dS K,
    dK = scale dS^T Q.

All arithmetic is float64 (numpy).  Rows of a head are processed in blocks only to bound memory;
every score row is complete inside its block, so a block size of N is the unblocked definition.
"""
from __future__ import annotations

import numpy as np

__all__ = ["scores", "softmax_rows", "block_grads", "forward", "forward_rows", "backward", "backward_group", "as64"]


def as64(x) -> np.ndarray:
    """Widen a torch tensor or numpy array (any float dtype) to a float64 numpy array."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray, causal: bool) -> np.ndarray:
    """S = scale * Q_rows K^T with causal masking (key j > query i -> -inf)."""
    s = scale * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Safe softmax of each row: returns P, row max m and row sum l of exp(S - m)."""
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(finite[:, None], np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def _lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    with np.errstate(divide="ignore"):
        return np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)


def _check(q, k, v):
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (B, N, d) != (Bk, Nk, dk) or v.shape != k.shape or Hkv < 1 or Hq % Hkv:
        raise ValueError(f"incompatible shapes q{q.shape} k{k.shape} v{v.shape}")
    return B, Hq, Hkv, N, d, Hq // Hkv


def forward_rows(q, k, v, causal: bool, scale: float, b: int, h: int, rows):
    """O and LSE of query head h of batch b for the given query rows (each row is independent)."""
    q, k, v = as64(q), as64(k), as64(v)
    B, Hq, Hkv, N, d, G = _check(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    g = h // G
    s = scores(q[b, h, rows], k[b, g], scale, rows, causal)
    p, m, l = softmax_rows(s)
    return p @ v[b, g], _lse(m, l)


def forward(q, k, v, causal: bool, scale: float, row_block: int | None = None):
    """O [B,Hq,N,d] and LSE [B,Hq,N] (natural log) in float64."""
    q, k, v = as64(q), as64(k), as64(v)
    B, Hq, Hkv, N, d, G = _check(q, k, v)
    rb = N if row_block is None else max(1, int(row_block))
    o = np.empty((B, Hq, N, d))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, N, rb):
                rows = np.arange(r0, min(N, r0 + rb))
                o[b, h, rows], lse[b, h, rows] = forward_rows(q, k, v, causal, scale, b, h, rows)
    return o, lse


def block_grads(p, do_rows, q_rows, kg, vg, scale: float):
    """Chain rule for a set of complete query rows: (dQ rows, dK part, dV part, D rows)."""
    dv_add = p.T @ do_rows                 # dV = P^T dO
    dp = do_rows @ vg.T                    # dP = dO V^T
    dd = (p * dp).sum(axis=1)              # D_i = sum_j P_ij dP_ij
    ds = p * (dp - dd[:, None])            # through the softmax
    dq_rows = scale * (ds @ kg)            # dQ = scale dS K
    dk_add = scale * (ds.T @ q_rows)       # dK = scale dS^T Q
    return dq_rows, dk_add, dv_add, dd


def backward_group(q, k, v, do, causal: bool, scale: float, b: int, g: int, row_block: int | None = None):
    """Gradients for K/V head g of batch b and its query heads.

    Returns (dq [G,N,d] for query heads g*G .. g*G+G-1, dk [N,d], dv [N,d], D [G,N]).
    P is recomputed here from Q and K; nothing from a forward pass is consumed.
    """
    q, k, v, do = as64(q), as64(k), as64(v), as64(do)
    B, Hq, Hkv, N, d, G = _check(q, k, v)
    rb = N if row_block is None else max(1, int(row_block))
    kg, vg = k[b, g], v[b, g]
    dq = np.zeros((G, N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    dsum = np.zeros((G, N))
    for hh in range(G):
        h = g * G + hh
        for r0 in range(0, N, rb):
            rows = np.arange(r0, min(N, r0 + rb))
            s = scores(q[b, h, rows], kg, scale, rows, causal)
            p, _, _ = softmax_rows(s)
            dq_rows, dk_add, dv_add, dd = block_grads(p, do[b, h, rows], q[b, h, rows], kg, vg, scale)
            dq[hh, rows] = dq_rows
            dk += dk_add
            dv += dv_add
            dsum[hh, rows] = dd
    return dq, dk, dv, dsum


def backward(q, k, v, do, causal: bool, scale: float, row_block: int | None = None):
    """dQ [B,Hq,N,d], dK, dV [B,Hkv,N,d] of L = <O, dO>, in float64."""
    q, k, v, do = as64(q), as64(k), as64(v), as64(do)
    B, Hq, Hkv, N, d, G = _check(q, k, v)
    dq = np.empty((B, Hq, N, d))
    dk = np.empty((B, Hkv, N, d))
    dv = np.empty((B, Hkv, N, d))
    for b in range(B):
        for g in range(Hkv):
            dq[b, g * G:(g + 1) * G], dk[b, g], dv[b, g], _ = backward_group(q, k, v, do, causal, scale, b, g, row_block)
    return dq, dk, dv
