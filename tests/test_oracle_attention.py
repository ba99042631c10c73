"""Pins for the fp64 attention oracle: values that the pages and the mathematics fix.

None of these re-types the oracle's formulas: they check hand-derived worked examples, closed
forms of special inputs, invariants of softmax attention, brute-force finite differences and an
independent library implementation (torch float64 SDPA / autograd).
"""
import numpy as np
import pytest
import torch

from golden_io import read_assignments
from oracle import attention as A
from oracle import online

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- hand-derived worked example
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_hand_example(mode):
    g = read_assignments("hand_attention_n3_d2.txt")
    q, k, v, do = (g[n][None, None] for n in ("q", "k", "v", "do"))
    causal = mode == "causal"
    o, lse = A.forward(q, k, v, causal, 1.0)
    np.testing.assert_allclose(o[0, 0], g[f"o.{mode}"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], g[f"lse.{mode}"], rtol=0, atol=1e-13)
    dq, dk, dv = A.backward(q, k, v, do, causal, 1.0)
    np.testing.assert_allclose(dv[0, 0], g[f"dv.{mode}"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq[0, 0], g[f"dq.{mode}"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk[0, 0], g[f"dk.{mode}"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_one_key_returns_v(causal):
    q, k, v = rand(2, 3, 1, 8), rand(2, 3, 1, 8), rand(2, 3, 1, 8)
    o, lse = A.forward(q, k, v, causal, 0.37)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.37 * (q * k).sum(-1), atol=1e-14)


def test_causal_row0_is_v0():
    q, k, v = rand(1, 2, 17, 16), rand(1, 2, 17, 16), rand(1, 2, 17, 16)
    o, lse = A.forward(q, k, v, True, 0.25)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_average_v(causal):
    N = 23
    q, k, v = np.zeros((1, 2, N, 8)), rand(1, 2, N, 8), rand(1, 2, N, 8)
    o, lse = A.forward(q, k, v, causal, 1.0)
    if causal:
        cnt = np.arange(1, N + 1)
        want = np.cumsum(v, axis=2) / cnt[None, None, :, None]
        want_lse = np.log(cnt)[None, None].repeat(2, 1)
    else:
        want = v.mean(axis=2, keepdims=True).repeat(N, axis=2)
        want_lse = np.full((1, 2, N), np.log(N))
    np.testing.assert_allclose(o, want, atol=1e-14)
    np.testing.assert_allclose(lse, want_lse, atol=1e-14)
    # Q = 0: dK = 0 (scores do not depend on K) and dV_j = sum_i P_ij dO_i with P uniform
    do = rand(1, 2, N, 8)
    dq, dk, dv = A.backward(q, k, v, do, causal, 1.0)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    if causal:
        w = 1.0 / np.arange(1, N + 1)
        want_dv = np.cumsum((do * w[None, None, :, None])[:, :, ::-1], axis=2)[:, :, ::-1]
    else:
        want_dv = do.mean(axis=2, keepdims=True).repeat(N, axis=2)
    np.testing.assert_allclose(dv, want_dv, atol=1e-13)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k = rand(9, 16), rand(9, 16)
    s = A.scores(q, k, 0.5, np.arange(9), causal)
    p, _, _ = A.softmax_rows(s)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(9, 1)] == 0.0)


def test_causal_future_keys_do_not_matter():
    q, k, v = rand(1, 1, 40, 16), rand(1, 1, 40, 16), rand(1, 1, 40, 16)
    o, lse = A.forward(q, k, v, True, 0.3)
    i = 17
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = rand(1, 1, 40 - i - 1, 16) * 5
    v2[:, :, i + 1:] = rand(1, 1, 40 - i - 1, 16) * 5
    o2, lse2 = A.forward(q, k2, v2, True, 0.3)
    assert np.array_equal(o[:, :, : i + 1], o2[:, :, : i + 1])
    assert np.array_equal(lse[:, :, : i + 1], lse2[:, :, : i + 1])
    assert not np.allclose(o[:, :, i + 1:], o2[:, :, i + 1:])


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v = rand(1, 2, 30, 8), rand(1, 2, 30, 8), rand(1, 2, 30, 8)
    u = rand(8)
    o, lse = A.forward(q, k, v, causal, 0.7)
    o2, lse2 = A.forward(q, k + u, v, causal, 0.7)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.7 * (q @ u), atol=1e-12)


def test_key_permutation_equivariance():
    q, k, v = rand(1, 1, 25, 8), rand(1, 1, 25, 8), rand(1, 1, 25, 8)
    perm = RNG.permutation(25)
    o, lse = A.forward(q, k, v, False, 0.5)
    o2, lse2 = A.forward(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(causal):
    B, Hq, Hkv, N, d = 2, 6, 2, 19, 8
    q, k, v, do = rand(B, Hq, N, d), rand(B, Hkv, N, d), rand(B, Hkv, N, d), rand(B, Hq, N, d)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)   # head h uses kv head h // G
    o, lse = A.forward(q, k, v, causal, 0.4)
    o2, lse2 = A.forward(q, kr, vr, causal, 0.4)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    dq, dk, dv = A.backward(q, k, v, do, causal, 0.4)
    dq2, dkr, dvr = A.backward(q, kr, vr, do, causal, 0.4)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dkr.reshape(B, Hkv, G, N, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dvr.reshape(B, Hkv, G, N, d).sum(2), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sums(causal):
    q, k, v, do = rand(1, 2, 33, 8), rand(1, 2, 33, 8), rand(1, 2, 33, 8), rand(1, 2, 33, 8)
    dq, dk, dv = A.backward(q, k, v, do, causal, 0.6)
    # rows of P sum to one -> sum_j dV_j = sum_i dO_i ; rows of dS sum to zero -> sum_j dK_j = 0
    np.testing.assert_allclose(dv.sum(2), do.sum(2), atol=1e-12)
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-12)
    # D_i = dO_i . O_i
    o, _ = A.forward(q, k, v, causal, 0.6)
    _, _, _, dsum = A.backward_group(q, k, v, do, causal, 0.6, 0, 1)
    np.testing.assert_allclose(dsum[0], (do[0, 1] * o[0, 1]).sum(-1), atol=1e-12)


def test_row_blocking_does_not_change_the_result():
    q, k, v, do = rand(1, 2, 50, 8), rand(1, 1, 50, 8), rand(1, 1, 50, 8), rand(1, 2, 50, 8)
    o1, l1 = A.forward(q, k, v, True, 0.5)
    o2, l2 = A.forward(q, k, v, True, 0.5, row_block=7)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)
    g1 = A.backward(q, k, v, do, True, 0.5)
    g2 = A.backward(q, k, v, do, True, 0.5, row_block=7)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-13)


# ---------------------------------------------------------------- brute force
def _loss(q, k, v, do, causal, scale):
    o, _ = A.forward(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("Hq,Hkv,N,d,causal", [
    (1, 1, 1, 4, False), (1, 1, 2, 4, True), (2, 1, 3, 4, False), (2, 2, 5, 8, True),
    (2, 1, 8, 4, True), (1, 1, 5, 8, False),
])
def test_finite_differences(Hq, Hkv, N, d, causal):
    rng = np.random.default_rng(N * 100 + d + 7 * Hq + causal)
    q, k, v, do = (rng.standard_normal(s) for s in [(1, Hq, N, d), (1, Hkv, N, d), (1, Hkv, N, d), (1, Hq, N, d)])
    scale = 0.8
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, causal, scale)
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-7, (name, err)


# ---------------------------------------------------------------- independent library
@pytest.mark.parametrize("Hq,Hkv,N,d,causal", [(4, 4, 65, 16, False), (4, 2, 65, 16, True), (8, 2, 100, 32, True)])
def test_against_torch_sdpa_float64(Hq, Hkv, N, d, causal):
    rng = np.random.default_rng(99)
    q, k, v, do = (rng.standard_normal(s) for s in [(2, Hq, N, d), (2, Hkv, N, d), (2, Hkv, N, d), (2, Hq, N, d)])
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                           enable_gqa=Hq != Hkv)
    ref.backward(torch.tensor(do))
    o, lse = A.forward(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ref.detach().numpy(), atol=1e-12)
    G = Hq // Hkv
    s = np.einsum("bhnd,bhmd->bhnm", q, np.repeat(k, G, axis=1)) * scale
    if causal:
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    ref_lse = torch.logsumexp(torch.tensor(s), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)
    dq, dk, dv = A.backward(q, k, v, do, causal, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------- the tiled online recurrence
@pytest.mark.parametrize("N,br,bc,causal", [(1, 4, 4, False), (37, 8, 16, False), (37, 8, 16, True),
                                            (64, 16, 16, True), (100, 32, 24, True), (100, 64, 128, False)])
def test_online_tiled_equals_definition(N, br, bc, causal):
    q, k, v = rand(1, 4, N, 16), rand(1, 2, N, 16), rand(1, 2, N, 16)
    o, lse = A.forward(q, k, v, causal, 0.25)
    o2, lse2, visited = online.forward_tiled(q, k, v, causal, 0.25, br, bc)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    # causal skipping visits exactly the key blocks that start at or before the last query row
    want = 0
    for r0 in range(0, N, br):
        last = min(N, r0 + br) - 1 if causal else N - 1
        want += last // bc + 1
    assert visited == want * 4


# ---------------------------------------------------------------- the pins catch planted mistakes
def _pins_pass():
    try:
        test_hand_example("full")
        test_hand_example("causal")
        test_one_key_returns_v(False)
        test_causal_row0_is_v0()
        test_gradient_sums(True)
        test_against_torch_sdpa_float64(4, 2, 65, 16, True)
    except AssertionError:
        return False
    return True


def test_pins_detect_planted_mistakes(monkeypatch):
    assert _pins_pass()
    good_scores, good_softmax, good_grads = A.scores, A.softmax_rows, A.block_grads

    def no_scale(q, k, scale, rows, causal):
        return good_scores(q, k, 1.0, rows, causal)

    def mask_off_by_one(q, k, scale, rows, causal):
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] >= rows[:, None], -np.inf, s)
        return s

    def transposed_scores(q, k, scale, rows, causal):
        return good_scores(q, k[:, ::-1], scale, rows, causal)

    def max_normalised(s):
        p, m, l = good_softmax(s)
        return p * l[:, None] / np.exp(0), m, l

    def wrong_sign_grads(p, do_rows, q_rows, kg, vg, scale):
        dq, dk, dv, dd = good_grads(p, do_rows, q_rows, kg, vg, scale)
        ds = p * (do_rows @ vg.T + dd[:, None])
        return scale * (ds @ kg), scale * (ds.T @ q_rows), dv, dd

    def dv_untransposed(p, do_rows, q_rows, kg, vg, scale):
        dq, dk, dv, dd = good_grads(p, do_rows, q_rows, kg, vg, scale)
        return dq, dk, p @ do_rows if p.shape[0] == p.shape[1] else dv * 1.01, dd

    for attr, bad in (("scores", no_scale), ("scores", mask_off_by_one), ("scores", transposed_scores),
                      ("softmax_rows", max_normalised), ("block_grads", wrong_sign_grads),
                      ("block_grads", dv_untransposed)):
        monkeypatch.setattr(A, attr, bad)
        assert not _pins_pass(), f"planted mistake {bad.__name__} went unnoticed"
        monkeypatch.undo()
    assert _pins_pass()
