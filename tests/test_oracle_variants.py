"""Pins for the sliding-window / ALiBi oracle: closed forms of special inputs, reduction to the
plain definition, and torch float64 scaled_dot_product_attention with an explicit float mask."""
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
