"""Pins for the sliding-window / ALiBi oracle: closed forms of special inputs, reduction to the
plain definition, and torch float64 scaled_dot_product_attention with an explicit float mask.
Backward: torch float64 autograd through that SDPA, central finite differences on tiny inputs,
the window-1 closed form (P = I), and the plain backward when there is neither window nor bias."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import variants as VA

RNG = np.random.default_rng(4242)


def rand(*shape):
    return RNG.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_no_window_no_slopes_is_the_plain_definition(causal):
    q, k, v = rand(2, 4, 19, 8), rand(2, 2, 19, 8), rand(2, 2, 19, 8)
    o, lse = VA.forward(q, k, v, causal, 0.3)
    o2, lse2 = A.forward(q, k, v, causal, 0.3)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    o3, lse3 = VA.forward(q, k, v, causal, 0.3, window=19, slopes=np.zeros(4))
    np.testing.assert_allclose(o3, o2, atol=1e-15)
    np.testing.assert_allclose(lse3, lse2, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_window_one_returns_own_value(causal):
    q, k, v = rand(1, 2, 13, 8), rand(1, 2, 13, 8), rand(1, 2, 13, 8)
    o, lse = VA.forward(q, k, v, causal, 0.7, window=1)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q * k).sum(-1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("W", [2, 5, 40])
def test_window_uniform_scores_average_the_band(causal, W):
    N = 23
    q, k, v = np.zeros((1, 1, N, 8)), rand(1, 1, N, 8), rand(1, 1, N, 8)
    o, lse = VA.forward(q, k, v, causal, 1.0, window=W)
    for i in range(N):
        lo = max(0, i - W + 1)
        hi = i if causal else min(N - 1, i + W - 1)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.log(hi - lo + 1), atol=1e-14)


def test_alibi_uniform_scores_geometric_weights():
    # q = 0: the weights of row i are r^(i-j), r = exp(-slope), over j <= i (causal)
    N, slope = 17, 0.37
    q, k, v = np.zeros((1, 1, N, 4)), rand(1, 1, N, 4), rand(1, 1, N, 4)
    o, lse = VA.forward(q, k, v, True, 1.0, slopes=np.array([slope]))
    r = np.exp(-slope)
    for i in range(N):
        w = r ** (i - np.arange(i + 1))
        np.testing.assert_allclose(o[0, 0, i], (w[:, None] * v[0, 0, :i + 1]).sum(0) / w.sum(), atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], np.log((1 - r ** (i + 1)) / (1 - r)), atol=1e-14)


@pytest.mark.parametrize("causal,W,alibi", [(False, 0, True), (True, 0, True), (True, 7, False), (False, 5, False),
                                            (True, 9, True), (False, 3, True)])
def test_against_torch_sdpa_float64(causal, W, alibi):
    B, Hq, Hkv, N, d = 2, 4, 2, 21, 16
    q, k, v = rand(B, Hq, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d)
    slopes = 2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq) if alibi else None
    o, lse = VA.forward(q, k, v, causal, 0.25, window=W, slopes=slopes)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    allowed = np.ones((N, N), bool)
    if causal:
        allowed &= j <= i
    if W:
        allowed &= (i - j < W) & ((j - i < W) | causal)
    bias = np.where(allowed, 0.0, -np.inf)[None, None].repeat(Hq, axis=1)
    if alibi:
        bias = bias - slopes[None, :, None, None] * np.abs(i - j)[None, None]
    G = Hq // Hkv
    tk = torch.from_numpy(np.repeat(k, G, axis=1))
    tv = torch.from_numpy(np.repeat(v, G, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), tk, tv,
                                                           attn_mask=torch.from_numpy(bias), scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    # and the logsumexp against torch's
    s = 0.25 * torch.from_numpy(q) @ tk.transpose(-1, -2) + torch.from_numpy(bias)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_rows_equal_the_full_forward():
    q, k, v = rand(1, 2, 30, 8), rand(1, 1, 30, 8), rand(1, 1, 30, 8)
    sl = np.array([0.1, 0.5])
    o, lse = VA.forward(q, k, v, True, 0.4, window=6, slopes=sl)
    for h in range(2):
        ro, rl = VA.forward_rows(q, k, v, True, 0.4, 6, sl, 0, h, [0, 5, 29])
        np.testing.assert_allclose(ro, o[0, h, [0, 5, 29]], atol=1e-15)
        np.testing.assert_allclose(rl, lse[0, h, [0, 5, 29]], atol=1e-15)


# ---- backward


def _torch_grads(q, k, v, do, causal, scale, W, slopes):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    allowed = np.ones((N, N), bool)
    if causal:
        allowed &= j <= i
    if W:
        allowed &= (i - j < W) & ((j - i < W) | causal)
    bias = np.where(allowed, 0.0, -np.inf)[None, None].repeat(Hq, axis=1)
    if slopes is not None:
        bias = bias - slopes[None, :, None, None] * np.abs(i - j)[None, None]
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk.repeat_interleave(G, dim=1),
                                                           tv.repeat_interleave(G, dim=1),
                                                           attn_mask=torch.from_numpy(bias), scale=scale)
    (out * torch.from_numpy(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal,W,alibi", [(False, 0, True), (True, 0, True), (True, 7, False), (False, 5, False),
                                            (True, 9, True), (False, 3, True)])
def test_backward_against_torch_autograd(causal, W, alibi):
    B, Hq, Hkv, N, d = 2, 4, 2, 21, 16
    q, k, v, do = rand(B, Hq, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, Hq, N, d)
    slopes = 2.0 ** (-8.0 * np.arange(1, Hq + 1) / Hq) if alibi else None
    got = VA.backward(q, k, v, do, causal, 0.25, window=W, slopes=slopes)
    ref = _torch_grads(q, k, v, do, causal, 0.25, W, slopes)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("causal,W", [(True, 3), (False, 2)])
def test_backward_finite_differences(causal, W):
    B, Hq, Hkv, N, d = 1, 2, 1, 6, 4
    q, k, v, do = rand(B, Hq, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, Hq, N, d)
    slopes = np.array([0.3, 0.05])
    scale, hh = 0.6, 1e-6
    got = VA.backward(q, k, v, do, causal, scale, window=W, slopes=slopes)

    def loss(qq, kk, vv):
        return float((VA.forward(qq, kk, vv, causal, scale, window=W, slopes=slopes)[0] * do).sum())

    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += hh
            xm[idx] -= hh
            a_p, a_m = [q, k, v], [q, k, v]
            a_p[which], a_m[which] = xp, xm
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * hh)
        np.testing.assert_allclose(got[which], num, rtol=1e-7, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_window_one_closed_form(causal):
    # window 1: each row sees only itself, P = I: dQ = dK = 0 and dV = the group sum of dO
    q, k, v, do = rand(1, 4, 9, 8), rand(1, 2, 9, 8), rand(1, 2, 9, 8), rand(1, 4, 9, 8)
    dq, dk, dv = VA.backward(q, k, v, do, causal, 0.5, window=1, slopes=np.array([0.1, 0.2, 0.3, 0.4]))
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0], do[0].reshape(2, 2, 9, 8).sum(1), atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_no_window_no_slopes_is_the_plain_backward(causal):
    q, k, v, do = rand(2, 4, 13, 8), rand(2, 1, 13, 8), rand(2, 1, 13, 8), rand(2, 4, 13, 8)
    got = VA.backward(q, k, v, do, causal, 0.3)
    ref = A.backward(q, k, v, do, causal, 0.3)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-13)
