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

MX recipe (the OCP Microscaling Formats specification, MXFP8 with E4M3
elements, cited as [OCP-MX]): blocks of 32 elements along the contraction
axis share one E8M0 scale 2^X with
    X     = floor(log2(amax)) - 8   (8: exponent of the largest power of two
                                     an E4M3 element holds), clamped to
                                     [-127, 127]; -127 when amax == 0
    code  = E4M3 round-to-nearest-even, saturated to +-448, of v * 2^-X
            (an exact scaling)
    value = decode(code) * 2^X;   stored scale byte = X + 127
"""

import math

import numpy as np

E4M3_MAX = 448.0


def _decode_definition(codes):
    """Value of each E4M3 code from the format's fields (float64; NaN for
    S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = s * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = s * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


_DECODE_TABLE = _decode_definition(np.arange(256))


def decode(codes):
    """Value of each E4M3 code (float64; NaN for S.1111.111): the definition
    above, evaluated once for all 256 codes and looked up."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


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


def _scales(amax):
    """(scale, inv) of an array of block maxima: the same fp32 divisions as
    ``block_scale``, element by element (NumPy's float32 division is the IEEE
    one), and 1 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    return scale, inv


def quantize_rows(x, block=128):
    """1 x ``block`` tiles along the last axis of x [M, K] (K % block == 0).
    Returns codes uint8 [M, K] and fp32 scales [M, K / block].  Every tile at
    once: amax per tile, ``block_scale``'s fp32 scale and inverse, one fp32
    product per element, then ``encode``."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % block == 0
    t = x.reshape(M, K // block, block)
    scale, inv = _scales(np.abs(t).max(axis=2) if M else np.zeros((0, K // block), np.float32))
    q = encode((t * inv[:, :, None]).astype(np.float32)).reshape(M, K)
    return q, scale


def quantize_blocks(w, block=128):
    """``block`` x ``block`` tiles of w [K, N] (both multiples of block).
    Returns codes uint8 [K, N] and fp32 scales [K / block, N / block]."""
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    assert K % block == 0 and N % block == 0
    t = w.reshape(K // block, block, N // block, block)
    scale, inv = _scales(np.abs(t).max(axis=(1, 3)))
    q = encode((t * inv[:, None, :, None]).astype(np.float32)).reshape(K, N)
    return q, scale


def dequantize_rows(q, s, block=128):
    return decode(q) * np.repeat(np.asarray(s, np.float64), block, axis=1)


def dequantize_blocks(q, s, block=128):
    s = np.asarray(s, np.float64)
    return decode(q) * np.repeat(np.repeat(s, block, axis=0), block, axis=1)


def to_bf16(a):
    """Round to the nearest bfloat16 (ties to even), returned as float32: the
    storage dtype of the tensors the fp8 quantizers read."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def padded_offsets(offsets, block=128):
    """Each group's row count rounded up to a multiple of ``block``."""
    offsets = np.asarray(offsets, dtype=np.int64)
    sizes = np.diff(offsets)
    padded = (sizes + block - 1) // block * block
    out = np.zeros(len(offsets), dtype=np.int64)
    out[1:] = np.cumsum(padded)
    return out


def quantize_token_tiles(x, offsets, block=128):
    """``block`` tokens x 1 tiles along the rows of x [M, K], per group of
    rows [offsets[g], offsets[g+1]), each group zero-padded to a multiple of
    ``block`` rows (the contraction axis of a weight gradient is the tokens).
    Returns codes uint8 [M_pad, K], fp32 scales [M_pad / block, K] and the
    padded offsets.  Padding rows are zeros, so they change no tile's amax
    and get code 0."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    poff = padded_offsets(offsets, block)
    M_pad = int(poff[-1])
    xp = np.zeros((M_pad, K), dtype=np.float32)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        xp[poff[g]:poff[g] + hi - lo] = x[lo:hi]
    t = xp.reshape(M_pad // block, block, K)
    scale, inv = _scales(np.abs(t).max(axis=1) if M_pad else np.zeros((0, K), np.float32))
    q = encode((t * inv[:, None, :]).astype(np.float32)).reshape(M_pad, K)
    return q, scale, poff


def dequantize_token_tiles(q, s, block=128):
    return decode(q) * np.repeat(np.asarray(s, np.float64), block, axis=0)


def layer_fp8(x, w_r, w13, w2, dout, k, score, renorm, logit_bias=None, shared=None,
              quantize=True, block=128, recipe="block", trace=None, z=None, capacity=None):
    """Forward and backward of the MoE layer with every expert-GEMM input
    quantized blockwise to E4M3 (the fp8 recipe above), computed as fp64
    grouped GEMMs on the dequantized values.

    Forward and dgrad operands use 1 x block tiles along their contraction
    axis (rows of X_perm, H, dY, dAB); weights use block x block blocks (the
    same blocks serve the transposed use in dgrad); weight-gradient operands
    use block-token x 1 tiles, each expert's rows zero-padded to a multiple
    of block.  The quantizers read bf16 tensors (the storage dtype of the
    activations), so a value is rounded to bf16 before it is quantized.
    Routing, permutation, SwiGLU and combine are exact (fp64, fp32 keys).
    ``quantize=False`` replaces every quantize/dequantize pair with the
    identity (the exact layer).  ``recipe="mx"``: MXFP8 instead (1 x 32
    blocks along every operand's contraction axis, E8M0 scales; a weight then
    has one quantization per GEMM that reads it).  Returns a dict of outputs
    and gradients.  ``trace``, if a dict, receives every GEMM's operands as
    fed to it (dequantized), keyed "<gemm>.A" / "<gemm>.B", together with the
    tensors they were quantized from ("src.<name>") and the padded offsets;
    recording changes nothing that is computed.  ``z`` may give the fp32 keys
    directly (by default they are computed with ``router_logits``).
    ``capacity`` drops what exceeds it (``apply_capacity``, the capacity-limited
    dropping of section 7, Load Balancing): a dropped (token, slot) pair has no
    row, adds nothing to the output and gets no gradient.
    """
    from . import moe_oracle as o

    mx = recipe == "mx"

    def q_rows(a):
        if not quantize:
            return o.f64(a)
        if mx:
            return dequantize_mx_rows(*quantize_mx_rows(to_bf16(a)))
        qq, ss = quantize_rows(to_bf16(a), block)
        return dequantize_rows(qq, ss, block)

    def q_weights(w, use="fwd"):
        if not quantize:
            return o.f64(w)
        if mx:
            out = []
            for wg in w:
                qf, sf, qd, sd = quantize_mx_weight(to_bf16(wg))
                out.append(dequantize_mx_rows(qf, sf).T if use == "fwd"
                           else dequantize_mx_rows(qd, sd))
            return np.stack(out)
        return np.stack([dequantize_blocks(*quantize_blocks(to_bf16(wg), block), block)
                         for wg in w])

    def q_tiles(a, offsets):
        """Returns the padded dequantized rows and the padded offsets."""
        if not quantize:
            return o.f64(a), np.asarray(offsets, np.int64)
        if mx:
            qq, ss, poff = quantize_mx_token_tiles(to_bf16(a), offsets)
            return dequantize_mx_token_tiles(qq, ss), poff
        qq, ss, poff = quantize_token_tiles(to_bf16(a), offsets, block)
        return dequantize_token_tiles(qq, ss, block), poff

    def rec(name, a):
        if trace is not None:
            trace[name] = a
        return a

    x = o.f64(x)
    T = x.shape[0]
    if z is None:
        z = o.router_logits(x, w_r, logit_bias)
    r = o.route(z, k, score, renorm)
    if capacity is not None:
        r = o.apply_capacity(r, capacity)
    off = r["offsets"]
    # a dropped slot (dst_row -1) reads and writes an extra all-zero row past
    # the kept rows, so combine, its backward and permute_bwd add nothing for it
    n_rows = int(off[-1])
    dst = np.where(r["dst_row"] < 0, n_rows, r["dst_row"])

    def zero_row(a):
        return np.concatenate([a, np.zeros((1, a.shape[1]))])

    w13d, w2d = rec("fwd1.B", q_weights(w13)), rec("fwd2.B", q_weights(w2))
    w13g, w2g = (q_weights(w13, "dgrad"), q_weights(w2, "dgrad")) if mx else (w13d, w2d)
    rec("dgrad1.B", w13g)
    rec("dgrad2.B", w2g)
    xp = rec("src.xp", o.permute(x, r["src_token"]))
    ab = o.grouped_gemm_fwd(rec("fwd1.A", q_rows(xp)), w13d, off)
    h = rec("src.h", o.swiglu(ab))
    y = o.grouped_gemm_fwd(rec("fwd2.A", q_rows(h)), w2d, off)
    ys = None
    if shared is not None:
        ws13d, ws2d = q_weights(np.asarray(shared[0])[None]), q_weights(np.asarray(shared[1])[None])
        ws13g, ws2g = ((q_weights(np.asarray(shared[0])[None], "dgrad"),
                        q_weights(np.asarray(shared[1])[None], "dgrad")) if mx else (ws13d, ws2d))
        rec("s.fwd1.B", ws13d)
        rec("s.fwd2.B", ws2d)
        rec("s.dgrad1.B", ws13g)
        rec("s.dgrad2.B", ws2g)
        all_rows = np.array([0, T])
        abs_ = o.grouped_gemm_fwd(rec("s.fwd1.A", q_rows(x)), ws13d, all_rows)
        hs = rec("src.hs", o.swiglu(abs_))
        ys = o.grouped_gemm_fwd(rec("s.fwd2.A", q_rows(hs)), ws2d, all_rows)
    out = o.unpermute_combine(zero_row(y), r["topk_w"], dst, ys)

    dout = o.f64(dout)
    dy, dw = o.unpermute_combine_bwd(dout, zero_row(y), r["topk_w"], dst)
    dy = dy[:n_rows]
    rec("src.dy", dy)
    dh = o.grouped_gemm_dgrad(rec("dgrad2.A", q_rows(dy)), w2g, off)
    dab = rec("src.dab", o.swiglu_bwd(dh, ab))
    dxp = o.grouped_gemm_dgrad(rec("dgrad1.A", q_rows(dab)), w13g, off)
    hp, poff = q_tiles(h, off)
    dyp, _ = q_tiles(dy, off)
    rec("poff", poff)
    dW2 = o.grouped_gemm_wgrad(rec("wgrad2.A", hp), rec("wgrad2.B", dyp), poff)
    xpp, _ = q_tiles(xp, off)
    dabp, _ = q_tiles(dab, off)
    dW13 = o.grouped_gemm_wgrad(rec("wgrad1.A", xpp), rec("wgrad1.B", dabp), poff)
    res = {}
    addends = []
    if shared is not None:
        dhs = o.grouped_gemm_dgrad(rec("s.dgrad2.A", q_rows(dout)), ws2g, all_rows)
        dabs = rec("src.dabs", o.swiglu_bwd(dhs, abs_))
        addends.append(o.grouped_gemm_dgrad(rec("s.dgrad1.A", q_rows(dabs)), ws13g, all_rows))
        hsp, ps = q_tiles(hs, all_rows)
        doutp, _ = q_tiles(dout, all_rows)
        xsp, _ = q_tiles(x, all_rows)
        dabsp, _ = q_tiles(dabs, all_rows)
        rec("s.poff", ps)
        res["dWs2"] = o.grouped_gemm_wgrad(rec("s.wgrad2.A", hsp), rec("s.wgrad2.B", doutp), ps)[0]
        res["dWs13"] = o.grouped_gemm_wgrad(rec("s.wgrad1.A", xsp), rec("s.wgrad1.B", dabsp), ps)[0]
    dz = o.route_bwd(z, r["topk_idx"], r["topk_w"], dw, score, renorm)
    dWr, dxr = o.router_logits_bwd(x, w_r, dz)
    addends.append(dxr)
    dx = o.permute_bwd(zero_row(dxp), dst, addends=tuple(addends))
    res.update(out=out, dx=dx, d_logits=dz, dW_r=dWr, dW13=dW13, dW2=dW2, z=z, route=r)
    return res


# ---------------------------------------------------------------- MXFP8 --
MX_BLOCK = 32
MX_EMAX = 8


def mx_exponent(amax):
    """Shared exponent X of MX blocks with max magnitude ``amax`` (a scalar or
    an array; exact: frexp gives floor(log2) for normal and subnormal values
    alike)."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(a)                     # a = m 2^e, 0.5 <= m < 1
    x = np.clip((e.astype(np.int64) - 1) - MX_EMAX, -127, 127)
    x = np.where(a == 0.0, -127, x)
    return int(x) if x.ndim == 0 else x


def mx_quantize_block(v):
    """Codes and scale bytes of blocks along the last axis of ``v`` (float32
    values; one block per row of that axis)."""
    v = np.asarray(v, dtype=np.float32)
    x = np.asarray(mx_exponent(np.max(np.abs(v), axis=-1)))
    scaled = np.ldexp(v.astype(np.float64), -x[..., None]).astype(np.float32)
    sb = (x + 127).astype(np.uint8)
    return encode(scaled), (int(sb) if sb.ndim == 0 else sb)


def mx_dequantize(q, sbytes):
    """decode(q) * 2^(byte - 127), sbytes broadcast to q's shape by the caller."""
    return decode(q) * np.ldexp(1.0, np.asarray(sbytes, np.int64) - 127)


def quantize_mx_rows(x):
    """1 x 32 blocks along the rows of x [M, K]: codes uint8 [M, K] and
    scale bytes uint8 [M, K / 32]."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    q, s = mx_quantize_block(x.reshape(M, K // MX_BLOCK, MX_BLOCK))
    return q.reshape(M, K), np.asarray(s, dtype=np.uint8).reshape(M, K // MX_BLOCK)


def dequantize_mx_rows(q, s):
    return mx_dequantize(q, np.repeat(s, MX_BLOCK, axis=1))


def quantize_mx_weight(w):
    """One expert's weight [K, N] for both GEMMs that read it: the forward
    contracts over K (blocks of 32 along K for each column: codes transposed
    [N, K], scales [N, K/32]); the data gradient contracts over N (blocks of
    32 along N for each row: codes [K, N], scales [K, N/32])."""
    w = np.asarray(w, dtype=np.float32)
    qf, sf = quantize_mx_rows(w.T)
    qd, sd = quantize_mx_rows(w)
    return qf, sf, qd, sd


def quantize_mx_token_tiles(x, offsets):
    """32-token x 1 blocks along the rows of x [M, K] per group of rows,
    each group zero-padded to a multiple of 128 rows: codes uint8 [M_pad, K],
    scale bytes uint8 [M_pad / 32, K], padded offsets."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    poff = padded_offsets(offsets, 128)
    M_pad = int(poff[-1])
    xp = np.zeros((M_pad, K), dtype=np.float32)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        xp[poff[g]:poff[g] + hi - lo] = x[lo:hi]
    qT, sT = quantize_mx_rows(xp.T) if M_pad else (np.zeros((K, 0), np.uint8),
                                                   np.zeros((K, 0), np.uint8))
    return qT.T.copy(), sT.T.copy(), poff


def dequantize_mx_token_tiles(q, s):
    return mx_dequantize(q, np.repeat(s, MX_BLOCK, axis=0))
