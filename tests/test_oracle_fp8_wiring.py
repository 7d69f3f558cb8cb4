"""Pins of the fp8 layer chain's wiring: which tensor each expert GEMM reads,
and along which tiles it was quantized.

The quantized layer ("Scalable Training of Mixture-of-Experts Models with
Megatron Core", section 5, Platform-specific recipes: 1 x 128 activation and
gradient tiles, 128 x 128 weight blocks) hands each GEMM dequantized operands.
A tile quantized with one scale is, by the format's definition, a set of E4M3
values times that scale with the largest magnitude code 448 (blockwise; the
scale is fp32(amax / 448)) or in [256, 448] (MX; the scale is 2^X).  So the
tiling an operand went through can be read off the operand itself: its tiles
along the right axis decompose exactly into E4M3 values times one scale, and
its tiles along the transposed axis (generically) do not.  That check needs
neither the chain's code nor the quantizers; it also catches an operand
quantized from the wrong tensor, which lands far from its source.

Readings checked (R14 and its MX counterpart): forward and data-gradient
operands in row tiles along their contraction axis; weights in 128 x 128
blocks (MX: 32 along K for the forward, along N for the data gradient);
weight-gradient operands in token tiles (128, MX: 32), each expert's rows
zero-padded to a multiple of 128.  The planted-mistake tests show that a
transposed tiling fails the check.
"""
import numpy as np
import pytest

import oracle
from oracle import fp8

E4M3_VALUES = np.unique(np.abs(fp8.decode(np.arange(256))[~np.isnan(fp8.decode(np.arange(256)))]))


def _tiles(a, tr, tc):
    """Tiles of tr x tc of a 2-D array (its sizes multiples of the tile), as
    [n_tiles, tr * tc]."""
    R, C = a.shape
    assert R % tr == 0 and C % tc == 0, (a.shape, tr, tc)
    return a.reshape(R // tr, tr, C // tc, tc).transpose(0, 2, 1, 3).reshape(-1, tr * tc)


def one_scale_per_tile(a, tr, tc, mx):
    """True when every tr x tc tile of ``a`` (2-D, or [G, R, C] per group) is
    E4M3 values times a single scale: amax / 448 (block recipe, the largest
    code 448) or 2^X with X = floor(log2 amax) - 8 (MX)."""
    a = np.asarray(a, np.float64)
    if a.ndim == 3:
        return all(one_scale_per_tile(g, tr, tc, mx) for g in a)
    t = _tiles(a, tr, tc)
    amax = np.abs(t).max(axis=1)
    live = amax > 0
    t, amax = t[live], amax[live]
    if mx:
        _, e = np.frexp(amax)
        scale = np.ldexp(1.0, e.astype(np.int64) - 1 - 8)
    else:
        scale = amax / 448.0
    codes = np.abs(t) / scale[:, None]
    return bool(np.isin(codes, E4M3_VALUES).all())


def _pad_rows(a, off, poff):
    out = np.zeros((int(poff[-1]), a.shape[1]))
    for g in range(len(off) - 1):
        out[poff[g]:poff[g] + off[g + 1] - off[g]] = a[off[g]:off[g + 1]]
    return out


def _close(deq, src, mx):
    """Within the E4M3 rounding of the bf16-rounded source: half a step
    (2^-4 relative; MX: 2^-3, as values in (448, 512) x 2^X saturate) plus
    the bf16 rounding, and the subnormal floor."""
    src = np.asarray(src, np.float64)
    rel = 2.0 ** -3 if mx else 2.0 ** -4
    tol = (rel + 2.0 ** -8) * np.abs(src) + 2.0 ** -9 * np.abs(src).max() / 448 * 8
    return bool((np.abs(deq - src) <= tol).all())


def wiring_failures(tr, mx, shared=True):
    """Every way the traced operands depart from the readings; [] if none."""
    blk = 32 if mx else 128
    tok = 32 if mx else 128
    rows = (1, blk)
    toks = (tok, 1)
    w_fwd = (32, 1) if mx else (128, 128)
    w_dgrad = (1, 32) if mx else (128, 128)
    off = tr["offsets"]
    poff = tr["poff"]
    expect = {
        "fwd1.A": (rows, toks, tr["src.xp"]), "fwd2.A": (rows, toks, tr["src.h"]),
        "dgrad2.A": (rows, toks, tr["src.dy"]), "dgrad1.A": (rows, toks, tr["src.dab"]),
        "wgrad2.A": (toks, rows, _pad_rows(tr["src.h"], off, poff)),
        "wgrad2.B": (toks, rows, _pad_rows(tr["src.dy"], off, poff)),
        "wgrad1.A": (toks, rows, _pad_rows(tr["src.xp"], off, poff)),
        "wgrad1.B": (toks, rows, _pad_rows(tr["src.dab"], off, poff)),
        "fwd1.B": (w_fwd, (1, blk), tr["w13"]), "fwd2.B": (w_fwd, (1, blk), tr["w2"]),
        "dgrad1.B": (w_dgrad, (blk, 1), tr["w13"]), "dgrad2.B": (w_dgrad, (blk, 1), tr["w2"]),
    }
    if shared:
        T = tr["src.x"].shape[0]
        s_off, s_poff = np.array([0, T]), tr["s.poff"]
        expect.update({
            "s.fwd1.A": (rows, toks, tr["src.x"]), "s.fwd2.A": (rows, toks, tr["src.hs"]),
            "s.dgrad2.A": (rows, toks, tr["src.dout"]), "s.dgrad1.A": (rows, toks, tr["src.dabs"]),
            "s.wgrad2.A": (toks, rows, _pad_rows(tr["src.hs"], s_off, s_poff)),
            "s.wgrad2.B": (toks, rows, _pad_rows(tr["src.dout"], s_off, s_poff)),
            "s.wgrad1.A": (toks, rows, _pad_rows(tr["src.x"], s_off, s_poff)),
            "s.wgrad1.B": (toks, rows, _pad_rows(tr["src.dabs"], s_off, s_poff)),
            "s.fwd1.B": (w_fwd, (1, blk), tr["ws13"][None]), "s.fwd2.B": (w_fwd, (1, blk), tr["ws2"][None]),
            "s.dgrad1.B": (w_dgrad, (blk, 1), tr["ws13"][None]),
            "s.dgrad2.B": (w_dgrad, (blk, 1), tr["ws2"][None]),
        })
    bad = []
    for name, (good, other, src) in expect.items():
        a = tr[name]
        if a.shape != np.shape(src):
            bad.append(f"{name}: shape {a.shape} vs source {np.shape(src)}")
            continue
        if not one_scale_per_tile(a, *good, mx):
            bad.append(f"{name}: not one scale per {good} tile")
        a_other = a
        if a.ndim == 2 and name.split(".")[-2].startswith(("fwd", "dgrad")):
            # token tiles of a row operand: over the same per-expert padding
            seg = (np.array([0, a.shape[0]]), tr["s.poff"]) if name.startswith("s.") else (off, poff)
            a_other = _pad_rows(a, *seg)
        if one_scale_per_tile(a_other, *other, mx):
            bad.append(f"{name}: also one scale per {other} tile (tiling not told apart)")
        if not _close(a, src, mx):
            bad.append(f"{name}: not the quantization of its source tensor")
    return bad


def _run(mx, shared=True, seed=3):
    from test_oracle_layer import _make
    x, w_r, w13, w2, b, sh, dout = _make(seed, T=300, d=256, E=4, k=2, f=128, fs=128, bias=True)
    if not shared:
        sh = None
    tr = {}
    fp8.layer_fp8(x, w_r, w13, w2, dout, 2, oracle.SIGMOID, True, logit_bias=b, shared=sh,
                  recipe="mx" if mx else "block", trace=tr)
    tr.update({"src.x": np.asarray(x, np.float64), "src.dout": np.asarray(dout, np.float64),
               "w13": np.asarray(w13, np.float64), "w2": np.asarray(w2, np.float64)})
    r = oracle.route(oracle.router_logits(x, w_r, b), 2, oracle.SIGMOID, True)
    tr["offsets"] = r["offsets"]
    if sh is not None:
        tr["ws13"], tr["ws2"] = np.asarray(sh[0], np.float64), np.asarray(sh[1], np.float64)
    return tr


@pytest.mark.parametrize("mx", [False, True], ids=["blockwise", "mxfp8"])
def test_layer_fp8_operands_follow_the_tilings(mx):
    """Every expert-GEMM operand of the quantized chain (routed and shared,
    forward and backward) carries one scale per tile of its reading's tiling,
    not of the transposed one, and is the quantization of the right tensor."""
    tr = _run(mx)
    assert wiring_failures(tr, mx) == []
    # ragged segments: the padded operands really are padded per expert
    assert (np.diff(tr["poff"]) % 128 == 0).all() and (np.diff(tr["offsets"]) % 128 != 0).any()


def test_tile_check_tells_tilings_apart():
    """The check itself: one row-quantized matrix passes as rows and fails as
    token tiles; a token-tile-quantized one the other way round; a 128 x 128
    block-quantized one fails as 1 x 128 rows."""
    rng = np.random.default_rng(1)
    a = fp8.to_bf16(rng.standard_normal((256, 256)) * rng.uniform(0.1, 10, (256, 1)))
    qr = fp8.dequantize_rows(*fp8.quantize_rows(a))
    assert one_scale_per_tile(qr, 1, 128, False) and not one_scale_per_tile(qr, 128, 1, False)
    q, s, _ = fp8.quantize_token_tiles(a, np.array([0, 256]))
    qt = fp8.dequantize_token_tiles(q, s)
    assert one_scale_per_tile(qt, 128, 1, False) and not one_scale_per_tile(qt, 1, 128, False)
    qb = fp8.dequantize_blocks(*fp8.quantize_blocks(a))
    assert one_scale_per_tile(qb, 128, 128, False) and not one_scale_per_tile(qb, 1, 128, False)
    qm = fp8.dequantize_mx_rows(*fp8.quantize_mx_rows(a))
    assert one_scale_per_tile(qm, 1, 32, True) and not one_scale_per_tile(qm, 32, 1, True)


# ---- planted mistakes (in the oracle, on the CPU): each must be caught ----

def _rows_instead_of_token_tiles(monkeypatch, mx):
    def quant(x, offsets, block=128):
        poff = fp8.padded_offsets(offsets, 128)
        xp = _pad_rows(np.asarray(x, np.float64), offsets, poff).astype(np.float32)
        deq = (fp8.dequantize_mx_rows(*fp8.quantize_mx_rows(xp)) if mx
               else fp8.dequantize_rows(*fp8.quantize_rows(xp)))
        return deq, None, poff
    if mx:
        monkeypatch.setattr(fp8, "quantize_mx_token_tiles", lambda x, off: quant(x, off))
        monkeypatch.setattr(fp8, "dequantize_mx_token_tiles", lambda q, s: q)
    else:
        monkeypatch.setattr(fp8, "quantize_token_tiles", quant)
        monkeypatch.setattr(fp8, "dequantize_token_tiles", lambda q, s, block=128: q)


@pytest.mark.parametrize("mx", [False, True], ids=["blockwise", "mxfp8"])
def test_planted_transposed_wgrad_tiling_is_caught(monkeypatch, mx):
    """Weight-gradient operands quantized in row tiles instead of token tiles
    (the plausible transposition) fail the check on all eight of them."""
    _rows_instead_of_token_tiles(monkeypatch, mx)
    bad = wiring_failures(_run(mx), mx)
    for name in ["wgrad1.A", "wgrad1.B", "wgrad2.A", "wgrad2.B"]:
        assert any(b.startswith(name + ":") for b in bad), (name, bad)
        assert any(b.startswith("s." + name + ":") for b in bad), (name, bad)


def test_planted_row_tiled_weights_are_caught(monkeypatch):
    """Weights quantized in 1 x 128 rows instead of 128 x 128 blocks."""
    monkeypatch.setattr(fp8, "quantize_blocks", lambda w, block=128: fp8.quantize_rows(w, block))
    monkeypatch.setattr(fp8, "dequantize_blocks",
                        lambda q, s, block=128: fp8.dequantize_rows(q, s, block))
    bad = wiring_failures(_run(False), False)
    for name in ["fwd1.B", "fwd2.B", "dgrad1.B", "dgrad2.B"]:
        assert any(b.startswith(name + ":") for b in bad), (name, bad)


def test_planted_swapped_mx_weight_blockings_are_caught(monkeypatch):
    """MX: the forward reading the weight blocked along N (the dgrad
    blocking) and the dgrad along K."""
    orig = fp8.quantize_mx_weight

    def swapped(w):
        qf, sf, qd, sd = orig(w)
        # forward operand built from the N-blocked codes, dgrad from the K-blocked ones
        deq_n = fp8.dequantize_mx_rows(qd, sd)             # [K, N], blocks along N
        deq_k = fp8.dequantize_mx_rows(qf, sf).T            # [K, N], blocks along K
        return deq_n.T, None, deq_k, None
    monkeypatch.setattr(fp8, "quantize_mx_weight", swapped)
    monkeypatch.setattr(fp8, "dequantize_mx_rows",
                        lambda q, s, _o=fp8.dequantize_mx_rows: q if s is None else _o(q, s))
    bad = wiring_failures(_run(True), True)
    for name in ["fwd1.B", "fwd2.B", "dgrad1.B", "dgrad2.B"]:
        assert any(b.startswith(name + ":") for b in bad), (name, bad)
