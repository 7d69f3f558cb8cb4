"""Pins of the oracle's grouped GEMMs (against one dense block-diagonal
product) and of its FP8 E4M3 codec (against the format's definition worked by
hand, torch's float8_e4m3fn cast, and exhaustive round trips)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from golden_io import read_sections


def _block_diag(A, offsets, G):
    M, K = A.shape
    out = np.zeros((M, G * K))
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        out[lo:hi, g * K:(g + 1) * K] = A[lo:hi]
    return out


@pytest.mark.parametrize("offsets", [[0, 5, 5, 12, 30], [0, 30], [0, 0, 0, 30, 30]])
def test_grouped_gemm_is_one_block_diagonal_product(offsets):
    rng = np.random.default_rng(0)
    G = len(offsets) - 1
    M, K, N = 30, 7, 9
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((G, K, N))
    dC = rng.standard_normal((M, N))
    Abd = _block_diag(A, offsets, G)
    Bst = B.reshape(G * K, N)
    np.testing.assert_allclose(oracle.grouped_gemm_fwd(A, B, offsets), Abd @ Bst, rtol=0, atol=1e-12)
    dAbd = dC @ Bst.T
    dA = oracle.grouped_gemm_dgrad(dC, B, offsets)
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        np.testing.assert_allclose(dA[lo:hi], dAbd[lo:hi, g * K:(g + 1) * K], rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.grouped_gemm_wgrad(A, dC, offsets).reshape(G * K, N),
                               Abd.T @ dC, rtol=0, atol=1e-12)


def test_swiglu_bwd_finite_differences():
    rng = np.random.default_rng(1)
    ab = rng.standard_normal((5, 8))
    dh = rng.standard_normal((5, 4))
    got = oracle.swiglu_bwd(dh, ab)
    eps = 1e-6
    num = np.zeros_like(ab)
    for pos in np.ndindex(ab.shape):
        p, m = ab.copy(), ab.copy()
        p[pos] += eps
        m[pos] -= eps
        num[pos] = ((oracle.swiglu(p) - oracle.swiglu(m)) * dh).sum() / (2 * eps)
    np.testing.assert_allclose(got, num, rtol=0, atol=1e-8)


def test_e4m3_landmarks():
    g = read_sections("e4m3_landmarks.txt")
    for code, val in g["decode"]:
        got = fp8.decode(int(code, 16))
        want = float(val)
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), code
    for val, code in g["encode"]:
        assert int(fp8.encode(np.float32(float(val)))) == int(code, 16), val


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])


def test_e4m3_encode_round_trip_and_torch_cast():
    vals = fp8.decode(np.arange(256))
    fin = ~np.isnan(vals)
    codes = np.arange(256)[fin]
    back = fp8.encode(vals[fin].astype(np.float32)).astype(np.int64)
    # -0.0 keeps its sign code
    np.testing.assert_array_equal(back, codes)
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1e-1, 1.0, 30.0, 200.0)])
    v = np.clip(v, -448, 448).astype(np.float32)
    # midpoints between neighbours exercise ties-to-even
    pos = np.sort(vals[fin & (vals >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.encode(v), ref)


def test_e4m3_saturates():
    v = np.array([449.0, 480.0, 1e6, np.inf, -np.inf, -1e6], dtype=np.float32)
    np.testing.assert_array_equal(fp8.encode(v), [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert fp8.encode(np.float32(np.nan)) == 0x7F


def test_blockwise_quantizers():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[1, :128] = 0.0
    q, s = fp8.quantize_rows(x)
    assert s.shape == (4, 2) and s[1, 0] == 1.0
    deq = fp8.dequantize_rows(q, s)
    # amax of each tile maps to +-448 exactly, and the relative error of
    # E4M3 with 3 mantissa bits is at most 2^-4 of the tile's amax.
    for i in range(4):
        for b in range(2):
            tile = x[i, b * 128:(b + 1) * 128]
            am = np.abs(tile).max()
            if am == 0:
                assert np.all(q[i, b * 128:(b + 1) * 128] == 0)
                continue
            assert np.abs(fp8.decode(q[i, b * 128:(b + 1) * 128])).max() == 448.0
            assert np.abs(deq[i, b * 128:(b + 1) * 128] - tile).max() <= am * 2.0 ** -4
    w = rng.standard_normal((256, 384)).astype(np.float32)
    qw, sw = fp8.quantize_blocks(w)
    assert sw.shape == (2, 3)
    assert np.abs(fp8.dequantize_blocks(qw, sw) - w).max() <= np.abs(w).max() * 2.0 ** -4


def test_token_tiles_equal_row_quantizer_on_transpose():
    """A 128-token x 1 tile is the row quantizer applied to the transposed
    tile; padding rows are zero codes."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 256)) * rng.uniform(0.01, 10, 256)).astype(np.float32)
    off = np.array([0, 0, 130, 131, 300])
    q, s, poff = fp8.quantize_token_tiles(x, off)
    np.testing.assert_array_equal(poff, [0, 0, 256, 384, 640])
    for g in range(4):
        lo, hi, plo = off[g], off[g + 1], poff[g]
        for b in range((hi - lo + 127) // 128):
            r0, r1 = lo + b * 128, min(hi, lo + b * 128 + 128)
            tile = np.zeros((128, 256), np.float32)
            tile[:r1 - r0] = x[r0:r1]
            qr, sr = fp8.quantize_rows(tile.T, block=128)
            np.testing.assert_array_equal(q[plo + b * 128:plo + b * 128 + 128].T, qr)
            np.testing.assert_array_equal(s[plo // 128 + b], sr[:, 0])


def test_fp8_layer_chain_without_quantization_is_the_exact_layer():
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, shared, dout = _make(5, T=40, d=12, E=4, k=2, f=10, fs=6, bias=True)
    for score, renorm in [(oracle.SIGMOID, True), (oracle.SOFTMAX, False)]:
        c = oracle.layer_forward(x, w_r, w13, w2, 2, score, renorm, logit_bias=b, shared=shared)
        g = oracle.layer_backward(c, dout)
        e = fp8.layer_fp8(x, w_r, w13, w2, dout, 2, score, renorm, logit_bias=b, shared=shared,
                          quantize=False)
        np.testing.assert_allclose(e["out"], c["out"], rtol=0, atol=1e-12)
        for name in ["dx", "d_logits", "dW_r", "dW13", "dW2", "dWs13", "dWs2"]:
            np.testing.assert_allclose(e[name], g[name], rtol=0, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("recipe", ["block", "mx"])
def test_fp8_layer_unquantized_with_capacity_is_the_exact_layer(recipe):
    """With capacity-limited dropping the grouped chain (kept rows only, dropped
    pairs skipped in combine and its backward) equals the per-token layer that
    skips the dropped pairs; the capacity is small enough that pairs drop."""
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, shared, dout = _make(8, T=48, d=12, E=4, k=2, f=10, fs=6, bias=True)
    cap = oracle.capacity_of(0.75, 48, 2, 4)
    for score, renorm in [(oracle.SIGMOID, True), (oracle.SOFTMAX, False)]:
        c = oracle.layer_forward(x, w_r, w13, w2, 2, score, renorm, logit_bias=b, shared=shared,
                                 capacity=cap)
        assert (c["route"]["dst_row"] < 0).sum() > 0
        g = oracle.layer_backward(c, dout)
        e = fp8.layer_fp8(x, w_r, w13, w2, dout, 2, score, renorm, logit_bias=b, shared=shared,
                          quantize=False, recipe=recipe, capacity=cap)
        np.testing.assert_array_equal(e["route"]["dst_row"], c["route"]["dst_row"])
        np.testing.assert_allclose(e["out"], c["out"], rtol=0, atol=1e-12)
        for name in ["dx", "d_logits", "dW_r", "dW13", "dW2", "dWs13", "dWs2"]:
            np.testing.assert_allclose(e[name], g[name], rtol=0, atol=1e-11, err_msg=name)


def test_fp8_layer_chain_close_to_exact_layer():
    """Sanity check of the chain's quantization error against the exact layer:
    E4M3 keeps 3 mantissa bits, so a few per cent of max|ref|, well below 20 %.
    (The 6e-2 bound applies between two quantized computations.)"""
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, shared, dout = _make(6, T=150, d=256, E=4, k=2, f=128, fs=128, bias=True)
    e = fp8.layer_fp8(x, w_r, w13, w2, dout, 2, oracle.SIGMOID, True, logit_bias=b, shared=shared)
    c = oracle.layer_forward(x, w_r, w13, w2, 2, oracle.SIGMOID, True, logit_bias=b, shared=shared)
    g = oracle.layer_backward(c, dout)
    rel = lambda a, r: np.abs(a - r).max() / np.abs(r).max()  # noqa: E731
    assert 1e-3 < rel(e["out"], c["out"]) < 0.2
    for name in ["dx", "dW13", "dW2", "dWs13", "dWs2"]:
        assert 1e-3 < rel(e[name], g[name]) < 0.2, name


def test_to_bf16_matches_torch():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(fp8.to_bf16(v), ref)


def test_mx_exponent_landmarks():
    """Shared exponent floor(log2(amax)) - 8 on landmarks: powers of two and
    their neighbours, fp32 subnormals, clamping, zero."""
    assert fp8.mx_exponent(0.0) == -127
    assert fp8.mx_exponent(256.0) == 0 and fp8.mx_exponent(511.99) == 0
    assert fp8.mx_exponent(255.99) == -1 and fp8.mx_exponent(512.0) == 1
    assert fp8.mx_exponent(1.0) == -8 and fp8.mx_exponent(np.float32(2.0 ** -100)) == -108
    assert fp8.mx_exponent(np.float32(2.0 ** -140)) == -127          # subnormal, clamped
    assert fp8.mx_exponent(np.float32(2.0 ** -119 * 1.5)) == -127    # -119 - 8 clamped
    assert fp8.mx_exponent(np.float32(3.0e38)) == 127 - 8


def test_mx_blocks_round_trip_exactly():
    """Blocks built from E4M3 codes and a shared exponent X, with the largest
    magnitude in [256, 448]: their MX quantization returns exactly those codes
    and X (the scale is the block's power of two, every value is
    representable).  Also: elements in (448, 512) x 2^X saturate to 448."""
    rng = np.random.default_rng(9)
    big = [c for c in range(0x7F) if 256 <= fp8.decode(c) <= 448]
    for _ in range(200):
        X = int(rng.integers(-100, 100))
        codes = rng.integers(0, 0x7F, 32).astype(np.uint8)
        codes[rng.integers(0, 32)] = rng.choice(big)
        codes |= (rng.integers(0, 2, 32) << 7).astype(np.uint8)
        v = (fp8.decode(codes) * 2.0 ** X).astype(np.float32)
        q, sb = fp8.mx_quantize_block(v)
        assert sb == X + 127
        np.testing.assert_array_equal(q, codes)
    v = np.zeros(32, np.float32)
    v[0], v[1] = 500.0 * 2.0 ** -20, 1.0 * 2.0 ** -20
    q, sb = fp8.mx_quantize_block(v)
    assert sb == -20 + 127 and q[0] == 0x7E and fp8.decode(q[1]) == 1.0


def test_mx_weight_layouts_and_layer_wiring():
    """The two MX quantizations of a weight cover it along K (forward) and
    along N (dgrad).  Each dequantizes to within half an E4M3 step (2^-4
    relative) of the weight, except elements above 448 x 2^X, which saturate
    (error below 1/8 relative: the block maximum is below 512 x 2^X).  And the
    MX layer chain with quantization switched off is the exact layer."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 96)).astype(np.float32)
    qf, sf, qd, sd = fp8.quantize_mx_weight(w)
    assert qf.shape == (96, 64) and sf.shape == (96, 2) and qd.shape == (64, 96) and sd.shape == (64, 3)
    for deq in (fp8.dequantize_mx_rows(qf, sf).T, fp8.dequantize_mx_rows(qd, sd)):
        err = np.abs(deq - w)
        assert (err <= np.abs(w) * 2.0 ** -3 + 2.0 ** -17 * np.abs(w).max()).all()
        assert np.median(err / np.abs(w)) < 2.0 ** -5
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, shared, dout = _make(5, T=40, d=12, E=4, k=2, f=10, fs=6, bias=True)
    c = oracle.layer_forward(x, w_r, w13, w2, 2, oracle.SOFTMAX, True, logit_bias=b, shared=shared)
    g = oracle.layer_backward(c, dout)
    r = fp8.layer_fp8(x, w_r, w13, w2, dout, 2, oracle.SOFTMAX, True, logit_bias=b, shared=shared,
                      quantize=False, recipe="mx")
    np.testing.assert_allclose(r["out"], c["out"], rtol=0, atol=1e-12)
    for n in ("dx", "d_logits", "dW_r", "dW13", "dW2", "dWs13", "dWs2"):
        np.testing.assert_allclose(r[n], g[n], rtol=0, atol=1e-11, err_msg=n)


def test_mx_token_tiles_are_32_token_blocks():
    """A 32-token x 1 MX block is the row quantizer applied to the transposed
    block; groups pad to 128 rows with zero codes and scale byte 0."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 64)) * rng.uniform(0.01, 10, 64)).astype(np.float32)
    off = np.array([0, 0, 130, 131, 300])
    q, s, poff = fp8.quantize_mx_token_tiles(x, off)
    np.testing.assert_array_equal(poff, [0, 0, 256, 384, 640])
    assert q.shape == (640, 64) and s.shape == (20, 64)
    for g in range(4):
        lo, hi, plo = off[g], off[g + 1], poff[g]
        for b in range((poff[g + 1] - plo) // 32):
            r0, r1 = lo + b * 32, min(hi, lo + b * 32 + 32)
            blk = np.zeros((32, 64), np.float32)
            if r1 > r0:
                blk[:r1 - r0] = x[r0:r1]
            qr, sr = fp8.quantize_mx_rows(blk.T)
            np.testing.assert_array_equal(q[plo + b * 32:plo + b * 32 + 32].T, qr)
            np.testing.assert_array_equal(s[plo // 32 + b], sr[:, 0])
    assert (s[9:12] == 0).all() and (q[288:384] == 0).all()      # group 2: one row, then padding


def test_mx_layer_chain_close_to_exact_layer():
    """MXFP8's power-of-two scales lose up to one more bit than an exact
    per-block scale: still a few per cent of max|ref|."""
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, shared, dout = _make(6, T=150, d=256, E=4, k=2, f=128, fs=128, bias=True)
    e = fp8.layer_fp8(x, w_r, w13, w2, dout, 2, oracle.SIGMOID, True, logit_bias=b, shared=shared,
                      recipe="mx")
    c = oracle.layer_forward(x, w_r, w13, w2, 2, oracle.SIGMOID, True, logit_bias=b, shared=shared)
    g = oracle.layer_backward(c, dout)
    rel = lambda a, r: np.abs(a - r).max() / np.abs(r).max()  # noqa: E731
    assert 1e-3 < rel(e["out"], c["out"]) < 0.2
    for name in ["dx", "dW13", "dW2", "dWs13", "dWs2"]:
        assert 1e-3 < rel(e[name], g[name]) < 0.2, name


def _brute_tile(v):
    """One tile by the definition, scalar by scalar: block_scale of its amax,
    then encode of each fp32 product."""
    scale, inv = fp8.block_scale(np.max(np.abs(v)))
    codes = np.array([fp8.encode(np.float32(e * inv)) for e in v.ravel()], np.uint8).reshape(v.shape)
    return codes, scale


def test_quantizers_equal_tile_by_tile_definition():
    """The whole-array quantizers give, tile for tile, the codes and scales of
    the definition applied to each tile alone (scalar fp32 arithmetic),
    including zero tiles, saturating values and subnormal codes."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((3, 256)) * np.array([[1e-3], [1.0], [300.0]])).astype(np.float32)
    x[0, 128:] = 0.0
    x[2, 5] = 3.0e38
    q, s = fp8.quantize_rows(x)
    for i in range(3):
        for b in range(2):
            c, sc = _brute_tile(x[i, b * 128:(b + 1) * 128])
            np.testing.assert_array_equal(q[i, b * 128:(b + 1) * 128], c)
            assert s[i, b] == sc
    w = (rng.standard_normal((256, 128)) * rng.uniform(1e-4, 10, (256, 1))).astype(np.float32)
    w[:128] = 0.0
    qw, sw = fp8.quantize_blocks(w)
    for i in range(2):
        c, sc = _brute_tile(w[i * 128:(i + 1) * 128])
        np.testing.assert_array_equal(qw[i * 128:(i + 1) * 128], c)
        assert sw[i, 0] == sc
    off = np.array([0, 3, 3, 140])
    xt = (rng.standard_normal((140, 2)) * 7).astype(np.float32)
    qt, st, poff = fp8.quantize_token_tiles(xt, off)
    assert list(poff) == [0, 128, 128, 384]
    for g, (lo, hi) in enumerate([(0, 3), (3, 140)]):
        plo = [0, 128][g]
        for b in range((hi - lo + 127) // 128):
            for col in range(2):
                v = np.zeros(128, np.float32)
                r1 = min(hi, lo + 128 * (b + 1))
                v[:r1 - lo - 128 * b] = xt[lo + 128 * b:r1, col]
                c, sc = _brute_tile(v)
                np.testing.assert_array_equal(qt[plo + 128 * b:plo + 128 * b + 128, col], c)
                assert st[plo // 128 + b, col] == sc
