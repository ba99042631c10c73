"""FP8 block quantisation with incoherent processing -- CPU reference.  TEST INFRASTRUCTURE.

Source: "FlashAttention-3: Fast and Accurate Attention with Asynchrony and Low-precision",
abstract: low-precision attention uses block quantisation (one scale per block) and incoherent
processing (a random orthogonal transform that spreads outliers before quantising).

Readings where the page is silent (each also recorded in the design notes):
  * format: OCP FP8 E4M3 ("e4m3fn": bias 7, no infinities, S.1111.111 is NaN, largest finite
    value 448, subnormals m * 2^-9); round to nearest even, saturating to +-448;
  * transform: x -> (x * s) H / sqrt(d) along the head dimension, with H the Sylvester Hadamard
    matrix of order d and s a vector of random signs; applied to Q and K only (it leaves
    Q K^T unchanged because M M^T = I), not to V;
  * one fp32 scale per (batch, head, block of 128 consecutive rows), scale = amax / 448
    (amax = largest magnitude in the block, all d columns; scale = 1 if amax = 0), and the
    stored code is e4m3(x / scale); or, as an option, the scale rounded up to a power of two:
    the smallest p = 2^e with 448 p >= amax (the E8M0 form of a block scale, which a
    block-scaled matrix multiply applies exactly; the page fixes one scale per block, not its
    value);
  * precision: the transform and the division run in float32 (the precision in which the GPU
    takes the same rounding decisions), the butterfly in the standard stage order
    h = 1, 2, 4, ..., d/2 with outputs (a + b, a - b).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3_MAX", "QBLOCK", "sylvester", "fwht_f32", "incoherent_f32", "e4m3_decode", "e4m3_encode",
    "block_quantize", "tensor_quantize", "dequantize", "pow2_scale",
]

E4M3_MAX = 448.0
QBLOCK = 128


def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1, float64."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis, in float32.

    Stage h (h = 1, 2, 4, ...) replaces each pair (a, b) = (x[i], x[i + h]) inside every block
    of 2h entries by (a + b, a - b).  Equals x @ sylvester(d) in exact arithmetic.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(lead + (d,))
        h *= 2
    return y


def incoherent_f32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """(x * signs) H / sqrt(d) in float32: signs, butterfly, then one multiply by fp32(1/sqrt(d))."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    s = np.asarray(signs).astype(np.float32)
    inv = np.float32(1.0 / np.sqrt(d))
    return (fwht_f32(x * s) * inv).astype(np.float32)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0 (exact, via frexp); 0 where a is 0 or not finite."""
    ok = np.isfinite(a) & (a > 0)
    _, ex = np.frexp(np.where(ok, a, 1.0))
    return np.where(ok, ex - 1, 0).astype(np.float64)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3 code (ties to even), saturating to +-448; NaN -> 0x7F; keeps the sign of zero.

    The quantum of a value of magnitude a is 2^(e-3) with e = max(floor(log2 a), -6)
    (e = -6 covers the subnormals, whose quantum 2^-9 equals the smallest normal's).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.clip(_floor_log2(a), -6, 8)
    quantum = 2.0 ** (e - 3)
    r = np.round(a / quantum) * quantum            # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)                    # saturate
    # encode the rounded magnitude (it may have moved up one binade)
    er = _floor_log2(r)
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, er + 7, 0)
    man_field = np.where(normal, r / 2.0 ** er * 8 - 8, r / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(man_field).astype(np.int64)
    code = np.where(r == 0, 0, code)
    code = code | np.where(np.signbit(x), 0x80, 0)     # IEEE: a negative value that rounds to 0 is -0
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def pow2_scale(amax: np.ndarray) -> np.ndarray:
    """Smallest power of two p with 448 p >= amax (1 where amax == 0), float32.

    With amax = m 2^k, m in [1, 2): amax / 448 = (m / 1.75) 2^(k - 8), and m / 1.75 lies in
    (1/2, 1] when m <= 1.75, in (1, 2) otherwise, so p = 2^(k - 8) or 2^(k - 7)."""
    a = np.asarray(amax, dtype=np.float64)
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = frac 2^ex, frac in [0.5, 1)
    m, k = 2.0 * frac, ex - 1                              # a = m 2^k, m in [1, 2)
    e = np.maximum(k - 8 + (m > 1.75).astype(np.int64), -149)   # at least the smallest float32
    return np.where(a > 0, np.ldexp(1.0, e), 1.0).astype(np.float32)


def block_quantize(x: np.ndarray, block: int = QBLOCK, pow2: bool = False):
    """x float32 [B,H,N,d] -> (codes uint8 [B,H,N,d], scales float32 [B,H,ceil(N/block)]);
    pow2: each scale rounded up to a power of two (pow2_scale)."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = -(-N // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for i in range(nb):
        blk = x[:, :, i * block:(i + 1) * block, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        if pow2:
            sc = pow2_scale(amax)
        else:
            sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        y = (blk / sc[:, :, None, None]).astype(np.float32)     # float32 division, correctly rounded
        codes[:, :, i * block:(i + 1) * block, :] = e4m3_encode(y)
        scales[:, :, i] = sc
    return codes, scales


def tensor_quantize(x: np.ndarray, block: int = QBLOCK):
    """The per-tensor scaling that the FlashAttention-3 abstract contrasts with block quantisation:
    one scale amax / 448 for the whole tensor (all heads, all rows), returned in the block layout
    (every entry equal) so that the same fp8 kernel consumes it."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    amax = np.float32(np.abs(x).max())
    sc = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    codes = e4m3_encode((x / sc).astype(np.float32))
    scales = np.full((B, H, -(-N // block)), sc, dtype=np.float32)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, block: int = QBLOCK) -> np.ndarray:
    """codes * scale of their block, float64."""
    vals = e4m3_decode(codes)
    rep = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :codes.shape[2]]
    return vals * rep[..., None]
