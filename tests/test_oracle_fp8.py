"""Pins for the fp8 quantisation reference: the e4m3 code table, the Hadamard transform, blocks."""
import numpy as np
import pytest
import torch

from golden_io import expr, read_rows
from oracle import attention as A
from oracle import fp8


def test_e4m3_golden_codes():
    for code, val in read_rows("e4m3_codes.txt", "decode"):
        got = fp8.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        want = expr(val)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)
    for val, code in read_rows("e4m3_codes.txt", "encode"):
        got = int(fp8.e4m3_encode(np.array([expr(val)]))[0])
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours).sum() == 2 and np.nanmax(ours) == 448.0


def test_e4m3_encode_against_torch_and_ties():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1e-1, 1, 30, 200)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    # every representable value and every midpoint between neighbours (ties)
    vals = np.unique(fp8.e4m3_decode(np.arange(256, dtype=np.uint8)))
    vals = vals[np.isfinite(vals)]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, vals.astype(np.float32), mids])
    ours = fp8.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # round trip of every finite code
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = fp8.e4m3_encode(fp8.e4m3_decode(codes))
    zero = (codes & 0x7F) == 0
    assert np.array_equal(back[~zero], codes[~zero])
    # saturation
    assert fp8.e4m3_encode(np.array([1e9, -1e9, 449.0]))[[0, 1, 2]].tolist() == [0x7E, 0xFE, 0x7E]


def test_sylvester_golden_and_orthogonal():
    h4 = np.array(read_rows("hadamard_4.txt"), dtype=np.float64)
    assert np.array_equal(fp8.sylvester(4), h4)
    for d in (1, 2, 8, 64, 128):
        h = fp8.sylvester(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        assert np.array_equal(h, h.T)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_fwht_equals_dense_product(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-50, 50, size=(7, d)).astype(np.float32)        # exact in float32
    assert np.array_equal(fp8.fwht_f32(x).astype(np.float64), x.astype(np.float64) @ fp8.sylvester(d))
    xf = rng.standard_normal((7, d)).astype(np.float32)
    np.testing.assert_allclose(fp8.fwht_f32(xf), xf.astype(np.float64) @ fp8.sylvester(d), rtol=0, atol=1e-4)


def test_incoherent_transform_preserves_scores_and_attention():
    rng = np.random.default_rng(3)
    d = 64
    q, k, v = (rng.standard_normal((1, 2, 40, d)) for _ in range(3))
    signs = np.where(rng.integers(0, 2, d) == 1, 1, -1)
    m = np.diag(signs.astype(np.float64)) @ fp8.sylvester(d) / np.sqrt(d)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-14)
    o, lse = A.forward(q, k, v, False, 0.125)
    o2, lse2 = A.forward(q @ m, k @ m, v, False, 0.125)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    # the float32 transform agrees with the exact one to float32 rounding
    xt = fp8.incoherent_f32(q.astype(np.float32), signs)
    np.testing.assert_allclose(xt, q @ m, rtol=0, atol=2e-5)


def test_block_quantize_properties():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 3, 300, 16)).astype(np.float32)
    x[0, 1, 128:256] = 0.0            # an all-zero block gets scale 1
    codes, scales = fp8.block_quantize(x)
    assert codes.shape == x.shape and scales.shape == (2, 3, 3)
    assert scales[0, 1, 1] == 1.0 and np.all(codes[0, 1, 128:256] == 0)
    for b, h, i in np.ndindex(2, 3, 3):
        blk = x[b, h, i * 128:(i + 1) * 128]
        if not np.any(blk):
            continue
        amax = np.abs(blk).max()
        assert scales[b, h, i] == np.float32(amax / np.float32(448.0))
        vals = np.abs(fp8.e4m3_decode(codes[b, h, i * 128:(i + 1) * 128]))
        assert vals.max() == 448.0          # the largest element lands on the top code
    deq = fp8.dequantize(codes, scales)
    # relative error of a normal e4m3 value is at most 2^-4; subnormals add an absolute 2^-10 * scale
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(scales, 128, axis=2)[:, :, :300, None] * 2.0 ** -10
    assert np.all(np.abs(deq - x) <= bound + 1e-12)


def test_tensor_quantize_properties():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 3, 300, 16)).astype(np.float32)
    x[1, 2, 17, 5] = -9.0                              # the tensor's amax lands on code -448
    codes, scales = fp8.tensor_quantize(x)
    assert scales.shape == (2, 3, 3) and np.all(scales == np.float32(9.0 / np.float32(448.0)))
    assert codes[1, 2, 17, 5] == 0xFE
    # one block covering the whole tensor is the same quantiser as block_quantize
    one = x[:1, :1, :128]
    c1, s1 = fp8.tensor_quantize(one)
    c2, s2 = fp8.block_quantize(one)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    deq = fp8.dequantize(codes, scales)
    bound = np.abs(x) * 2.0 ** -4 + float(scales[0, 0, 0]) * 2.0 ** -10
    assert np.all(np.abs(deq - x) <= bound + 1e-12)
    assert np.all(fp8.tensor_quantize(np.zeros((1, 1, 5, 4), np.float32))[1] == 1.0)


def test_pow2_scale_worked_values_and_definition():
    """The power-of-two block scale is the smallest p = 2^e with 448 p >= amax: worked values, then
    the definition checked by brute force over a wide range of magnitudes."""
    worked = {448.0: 1.0, 449.0: 2.0, 224.0: 0.5, 224.00002: 1.0, 447.99997: 1.0, 896.0: 2.0, 3.5: 2.0 ** -7,
              1.0: 2.0 ** -8, 0.0: 1.0}
    for a, p in worked.items():
        assert fp8.pow2_scale(np.float32(a)) == np.float32(p), (a, p)
    rng = np.random.default_rng(7)
    a = (np.exp(rng.uniform(-60, 60, size=20000)) * rng.uniform(0.5, 2.0, size=20000)).astype(np.float32)
    a = np.concatenate([a, (448.0 * np.ldexp(1.0, np.arange(-100, 100))).astype(np.float32)])
    p = fp8.pow2_scale(a).astype(np.float64)
    _, ex = np.frexp(p)
    assert np.all(np.frexp(p)[0] == 0.5)                  # a power of two
    assert np.all(448.0 * p >= a)                          # large enough
    assert np.all(448.0 * p / 2 < a)                       # and the smallest such


def test_block_quantize_pow2():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 2, 300, 16)).astype(np.float32) * 3
    x[0, 1, :128] = 0.0
    codes, scales = fp8.block_quantize(x, pow2=True)
    c_amax, s_amax = fp8.block_quantize(x)
    assert scales[0, 1, 0] == 1.0 and np.all(codes[0, 1, :128] == 0)
    for b, h, i in np.ndindex(1, 2, 3):
        blk = x[b, h, i * 128:(i + 1) * 128]
        if not np.any(blk):
            continue
        assert scales[b, h, i] == fp8.pow2_scale(np.abs(blk).max())
        # dividing by a power of two is exact, so the codes are the rounding of x / scale itself
        assert np.array_equal(codes[b, h, i * 128:(i + 1) * 128],
                              fp8.e4m3_encode(blk.astype(np.float64) / float(scales[b, h, i])))
        # the block's largest element lands in the top binade (224, 448]
        top = np.abs(fp8.e4m3_decode(codes[b, h, i * 128:(i + 1) * 128])).max()
        assert 224.0 <= top <= 448.0
    deq = fp8.dequantize(codes, scales)
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(scales, 128, axis=2)[:, :, :300, None] * 2.0 ** -10
    assert np.all(np.abs(deq - x) <= bound + 1e-12)
