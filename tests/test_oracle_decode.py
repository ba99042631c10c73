"""Pins for the decoding oracle (few query rows, long key sequence; key splits and their merge).

Closed forms of special inputs, invariants, an independent library routine (torch float64
scaled_dot_product_attention with an explicit mask) and the exactness of the logsumexp merge
against the unsplit definition.
"""
import numpy as np
import pytest
import torch

from oracle import decode as DC

RNG = np.random.default_rng(777)


def rand(*shape):
    return RNG.standard_normal(shape)


def test_single_query_single_key_is_v():
    q, k, v = rand(2, 4, 1, 8), rand(2, 2, 1, 8), rand(2, 2, 1, 8)
    o, lse = DC.forward(q, k, v, True, 0.3)
    kk = np.repeat(k, 2, axis=1)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=1), atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q * kk).sum(-1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_average_the_visible_values(causal):
    # every key equal: all visible keys get the same weight, LSE = s + ln(#visible)
    Nq, Nk = 3, 11
    q = rand(1, 2, Nq, 8)
    k = np.broadcast_to(rand(1, 1, 1, 8), (1, 1, Nk, 8)).copy()
    v = rand(1, 1, Nk, 8)
    o, lse = DC.forward(q, k, v, causal, 0.5)
    for i in range(Nq):
        n = (Nk - Nq + i + 1) if causal else Nk
        want = v[0, 0, :n].mean(axis=0)
        s = 0.5 * (q[0, :, i] @ k[0, 0, 0])
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(want, (2, 8)), atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], s + np.log(n), atol=1e-13)


def test_causal_rows_ignore_keys_after_their_position():
    Nq, Nk = 4, 20
    q, k, v = rand(1, 1, Nq, 8), rand(1, 1, Nk, 8), rand(1, 1, Nk, 8)
    o, lse = DC.forward(q, k, v, True, 0.4)
    for i in range(Nq):
        last = Nk - Nq + i                      # the row's position: keys after it are invisible
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, last + 1:] = rand(Nk - last - 1, 8) * 5
        v2[0, 0, last + 1:] = rand(Nk - last - 1, 8) * 5
        o2, lse2 = DC.forward(q, k2, v2, True, 0.4)
        assert np.array_equal(o2[0, 0, i], o[0, 0, i]) and lse2[0, 0, i] == lse[0, 0, i]


@pytest.mark.parametrize("Hq,Hkv,Nq,Nk,causal", [(2, 2, 1, 9, False), (4, 2, 3, 17, True), (8, 1, 4, 33, True),
                                                  (2, 1, 5, 5, True)])
def test_against_torch_sdpa_float64(Hq, Hkv, Nq, Nk, causal):
    d = 16
    q, k, v = rand(2, Hq, Nq, d), rand(2, Hkv, Nk, d), rand(2, Hkv, Nk, d)
    o, _ = DC.forward(q, k, v, causal, 0.31)
    G = Hq // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(np.repeat(k, G, axis=1))
    tv = torch.from_numpy(np.repeat(v, G, axis=1))
    mask = None
    if causal:   # bottom-right: row i sees keys j <= Nk - Nq + i
        mask = torch.from_numpy(np.arange(Nk)[None, :] <= (np.arange(Nq) + Nk - Nq)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.31)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_splits_equals_the_definition(splits, causal):
    Nq, Nk = 3, 40
    q, k, v = rand(2, 4, Nq, 8), rand(2, 2, Nk, 8), rand(2, 2, Nk, 8)
    o, lse = DC.forward(q, k, v, causal, 0.45)
    parts = DC.split_partials(q, k, v, causal, 0.45, DC.split_bounds(Nk, splits))
    mo, mlse = DC.merge(parts)
    np.testing.assert_allclose(mo, o, atol=1e-13)
    np.testing.assert_allclose(mlse, lse, atol=1e-13)
    # the merge does not depend on the order of the parts
    ro, rlse = DC.merge(parts[::-1])
    np.testing.assert_allclose(ro, mo, atol=1e-14)
    np.testing.assert_allclose(rlse, mlse, atol=1e-14)


def test_empty_and_invisible_splits_contribute_nothing():
    Nq, Nk = 2, 16
    q, k, v = rand(1, 1, Nq, 8), rand(1, 1, Nk, 8), rand(1, 1, Nk, 8)
    o, lse = DC.forward(q, k, v, True, 0.5)
    # the last key is seen only by the last row: for row 0 that split is empty (LSE -inf)
    parts = DC.split_partials(q, k, v, True, 0.5, [(0, 15), (15, 16), (16, 16)])
    assert np.isneginf(parts[1][1][0, 0, 0]) and np.all(parts[1][0][0, 0, 0] == 0)
    assert np.all(np.isneginf(parts[2][1]))
    mo, mlse = DC.merge(parts)
    np.testing.assert_allclose(mo, o, atol=1e-13)
    np.testing.assert_allclose(mlse, lse, atol=1e-13)


def test_split_bounds_cover_the_keys():
    for nk, s in [(1, 1), (10, 3), (128, 7), (1000, 16)]:
        b = DC.split_bounds(nk, s)
        assert b[0][0] == 0 and b[-1][1] == nk and all(b[i][1] == b[i + 1][0] for i in range(s - 1))
