"""FP8 E4M3 codec and blockwise quantizers -- TEST INFRASTRUCTURE ONLY.

Encoding: the OCP 8-bit Floating Point specification's E4M3 format ("FN":
bias 7, no infinities, only S.1111.111 is NaN, largest finite 448), cited as
[OCP-FP8].  Blockwise scaling follows [MCore-MoE] section 5 ("Platform-specific
recipes"): 1x128 tiles for activations and gradients, 128x128 blocks for
weights.  The scale arithmetic is fp32 (read where the page is silent):
    amax  = max |v| over the block (v exactly representable in fp32)
    scale = fp32(amax / 448), or 1.0 when amax == 0
    inv   = fp32(448 / amax), or 1.0 when amax == 0
    code  = E4M3 round-to-nearest-even, saturated to +-448, of fp32(v * inv)
    value = decode(code) * scale
"""

import numpy as np

E4M3_MAX = 448.0


def decode(codes):
    """Value of each E4M3 code (float64; NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = s * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = s * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES)


def encode(v):
    """Nearest E4M3 code to each fp32 value, ties to the even code, with
    magnitudes beyond 448 saturated to 448 and NaN mapped to 0x7F.

    Codes of one sign are ordered like their magnitudes, so the nearest value
    is one of the two bracketing table entries; on an exact midpoint the one
    whose code (hence mantissa) is even is taken.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    nan = np.isnan(v)
    sign = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(sign, code | 0x80, code)
    return np.where(nan, 0x7F, code).astype(np.uint8)


def block_scale(amax):
    """(scale, inv) for a block with max magnitude ``amax``, fp32 arithmetic."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0), np.float32(1.0)
    # numpy float32 scalar division is one IEEE fp32 division (nearest even)
    scale = np.float32(amax / np.float32(E4M3_MAX))
    inv = np.float32(np.float32(E4M3_MAX) / amax)
    return scale, inv


def quantize_rows(x, block=128):
    """1 x ``block`` tiles along the last axis of x [M, K] (K % block == 0).
    Returns codes uint8 [M, K] and fp32 scales [M, K / block]."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % block == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // block), dtype=np.float32)
    for i in range(M):
        for b in range(K // block):
            v = x[i, b * block:(b + 1) * block]
            scale, inv = block_scale(np.max(np.abs(v)))
            q[i, b * block:(b + 1) * block] = encode((v * inv).astype(np.float32))
            s[i, b] = scale
    return q, s


def quantize_blocks(w, block=128):
    """``block`` x ``block`` tiles of w [K, N] (both multiples of block).
    Returns codes uint8 [K, N] and fp32 scales [K / block, N / block]."""
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    assert K % block == 0 and N % block == 0
    q = np.empty((K, N), dtype=np.uint8)
    s = np.empty((K // block, N // block), dtype=np.float32)
    for i in range(K // block):
        for j in range(N // block):
            v = w[i * block:(i + 1) * block, j * block:(j + 1) * block]
            scale, inv = block_scale(np.max(np.abs(v)))
            q[i * block:(i + 1) * block, j * block:(j + 1) * block] = encode((v * inv).astype(np.float32))
            s[i, j] = scale
    return q, s


def dequantize_rows(q, s, block=128):
    return decode(q) * np.repeat(np.asarray(s, np.float64), block, axis=1)


def dequantize_blocks(q, s, block=128):
    s = np.asarray(s, np.float64)
    return decode(q) * np.repeat(np.repeat(s, block, axis=0), block, axis=1)
