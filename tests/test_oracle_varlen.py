"""Pins for the packed variable-length oracle: one sequence is the plain definition, sequences do
not see each other, a one-token sequence returns its value, and torch float64 SDPA with a
block-diagonal mask over the packed rows agrees."""
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
