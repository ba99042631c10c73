"""Pins for the packed variable-length oracle: one sequence is the plain definition, sequences do
not see each other, a one-token sequence returns its value, and torch float64 SDPA with a
block-diagonal mask over the packed rows agrees.  Backward: torch float64 autograd through that
masked SDPA, central finite differences of L = <O, dO> on tiny packed inputs, gradients that do
not cross sequences, and closed forms (a one-token sequence has dQ = dK = 0 and dV = the group
sum of its dO)."""
import numpy as np
import pytest
import torch

from attn_inputs import draw_varlen
from oracle import attention as A
from oracle import varlen as VL


@pytest.mark.parametrize("causal", [False, True])
def test_single_sequence_is_the_plain_definition(causal):
    q, k, v, cu = draw_varlen([37], 4, 2, 8, seed=1)
    o, lse = VL.forward(q, k, v, cu, causal, 0.3)
    o2, lse2 = A.forward(q[None], k[None], v[None], causal, 0.3)
    assert np.array_equal(o, o2[0]) and np.array_equal(lse, lse2[0])


@pytest.mark.parametrize("causal", [False, True])
def test_sequences_do_not_see_each_other(causal):
    lens = [5, 0, 11, 1, 7]
    q, k, v, cu = draw_varlen(lens, 2, 1, 8, seed=2)
    o, lse = VL.forward(q, k, v, cu, causal, 0.5)
    # change every token outside sequence 2: its rows stay bit for bit
    s0, s1 = cu[2], cu[3]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, :s0] *= -3.0
        x[:, s1:] += 1.0
    o2, lse2 = VL.forward(q2, k2, v2, cu, causal, 0.5)
    assert np.array_equal(o2[:, s0:s1], o[:, s0:s1]) and np.array_equal(lse2[:, s0:s1], lse[:, s0:s1])
    # the one-token sequence returns its value
    t = cu[3]
    np.testing.assert_allclose(o[:, t], np.repeat(v[:, t], 2, axis=0), atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_block_diagonal(causal):
    lens = [9, 3, 0, 14]
    Hq, Hkv, d = 4, 2, 16
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, d, seed=3)
    o, lse = VL.forward(q, k, v, cu, causal, 0.25)
    T = int(cu[-1])
    seg = np.repeat(np.arange(len(lens)), lens)
    allowed = seg[:, None] == seg[None, :]
    if causal:
        allowed &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    G = Hq // Hkv
    tq = torch.from_numpy(q.astype(np.float64))
    tk = torch.from_numpy(np.repeat(k, G, axis=0).astype(np.float64))
    tv = torch.from_numpy(np.repeat(v, G, axis=0).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(allowed), scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    s = 0.25 * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~torch.from_numpy(allowed), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def _torch_block_diag_grads(q, k, v, do, lens, causal, scale):
    """dQ, dK, dV by torch float64 autograd through SDPA with a block-diagonal (per-sequence) mask;
    K/V repeated over each query-head group and the repeats summed back."""
    T = int(sum(lens))
    seg = np.repeat(np.arange(len(lens)), lens)
    allowed = seg[:, None] == seg[None, :]
    if causal:
        allowed &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    Hq, Hkv = q.shape[0], k.shape[0]
    G = Hq // Hkv
    tq = torch.from_numpy(q.astype(np.float64)).requires_grad_()
    tk = torch.from_numpy(k.astype(np.float64)).requires_grad_()
    tv = torch.from_numpy(v.astype(np.float64)).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=0), tv.repeat_interleave(G, dim=0), attn_mask=torch.from_numpy(allowed),
        scale=scale)
    (out * torch.from_numpy(do.astype(np.float64))).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_against_torch_autograd_block_diagonal(causal):
    lens = [9, 3, 0, 14, 1]
    Hq, Hkv, d = 4, 2, 16
    q, k, v, cu = draw_varlen(lens, Hq, Hkv, d, seed=4)
    do = np.random.default_rng(5).standard_normal(q.shape)
    gq, gk, gv = VL.backward(q, k, v, do, cu, causal, 0.25)
    rq, rk, rv = _torch_block_diag_grads(q, k, v, do, lens, causal, 0.25)
    for a, b in ((gq, rq), (gk, rk), (gv, rv)):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    lens = [3, 1, 4]
    q, k, v, cu = draw_varlen(lens, 2, 1, 4, seed=6)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    do = np.random.default_rng(7).standard_normal(q.shape)
    scale, h = 0.7, 1e-6
    gq, gk, gv = VL.backward(q, k, v, do, cu, causal, scale)

    def loss(qq, kk, vv):
        return float((VL.forward(qq, kk, vv, cu, causal, scale)[0] * do).sum())

    for x, g, which in ((q, gq, 0), (k, gk, 1), (v, gv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-7, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_does_not_cross_sequences(causal):
    lens = [6, 0, 5, 1, 8]
    q, k, v, cu = draw_varlen(lens, 2, 2, 8, seed=8)
    do = np.random.default_rng(9).standard_normal(q.shape)
    gq, gk, gv = VL.backward(q, k, v, do, cu, causal, 0.4)
    s0, s1 = cu[2], cu[3]
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for x in (q2, k2, v2, do2):
        x[:, :s0] *= -2.0
        x[:, s1:] -= 0.5
    hq, hk, hv = VL.backward(q2, k2, v2, do2, cu, causal, 0.4)
    for a, b in ((gq, hq), (gk, hk), (gv, hv)):
        assert np.array_equal(a[:, s0:s1], b[:, s0:s1])
    # one-token sequence (rows cu[3]): P = 1, so dQ = dK = 0 and dV = the sum of its dO over the group
    t = cu[3]
    assert np.abs(gq[:, t]).max() < 1e-15 and np.abs(gk[:, t]).max() < 1e-15
    np.testing.assert_allclose(gv[:, t], do[:, t], atol=1e-15)


def test_backward_rows_outside_every_sequence_are_zero():
    lens = [4, 5]
    q, k, v, cu = draw_varlen(lens + [3], 2, 1, 8, seed=10)    # 3 trailing rows
    do = np.random.default_rng(11).standard_normal(q.shape)
    gq, gk, gv = VL.backward(q, k, v, do, cu[:-1], True, 0.5)
    assert not gq[:, 9:].any() and not gk[:, 9:].any() and not gv[:, 9:].any()
