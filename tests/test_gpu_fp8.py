"""FP8 (E4M3, blockwise fp32 scales) path against the oracle.

Quantizers: codes and scales bit-exact against oracle.fp8 on the same bf16
inputs.  GEMMs: the GPU consumes the oracle's own codes and scales (put in the
GEMM's layouts) and must match an fp64 grouped GEMM on the dequantized values
within 6e-2 (observed ~1e-3: products of codes are exact, the sums fp32).
Layer: MoELayer in fp8 mode against oracle.fp8.layer_fp8 (the oracle quantizes
at every expert-GEMM input itself) within 6e-2."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from routing_grouped_gemm_router_amd import abi, inputs
from routing_grouped_gemm_router_amd.layer import MoELayer
from gpu_util import TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16_data(shape, seed, special=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[-1], generator=g) * 2)
    if special:
        flat = x.view(-1, x.shape[-1])
        flat[0, :128] = 0.0                                   # all-zero block
        flat[1, :128] = torch.tensor([448.0, 1.0625, 1.1875, -1.0625, 0.0009765625, 3 * 2.0 ** -10]
                                     + [0.5] * 122)            # ties at scale 1
        flat[2, :128] = 1e-30                                 # tiny values
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,K", [(300, 512), (1000, 7168), (1, 128)])
def test_quant_rows_bit_exact(gpu, M, K):
    x = _bf16_data((M, K), 1, special=M >= 3)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    sT = torch.empty((K // 128, M), dtype=torch.float32, device=DEV)
    abi.moe_quant_fp8_rows(x.to(DEV), q, sT)
    rq, rs = fp8.quantize_rows(x.float().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(sT.cpu().numpy().T, rs)


@pytest.mark.parametrize("G,K,N", [(3, 256, 384), (2, 7168, 256)])
def test_quant_weights_bit_exact(gpu, G, K, N):
    w = _bf16_data((G, K, N), 2) * 0.05
    w[0, :128, :128] = 0.0
    q = torch.empty((G, K, N), dtype=torch.uint8, device=DEV)
    sf = torch.empty((G, K // 128, N), dtype=torch.float32, device=DEV)
    sd = torch.empty((G, N // 128, K), dtype=torch.float32, device=DEV)
    abi.moe_quant_fp8_weights(w.to(DEV), q, sf, sd)
    for g in range(G):
        rq, rs = fp8.quantize_blocks(w[g].float().numpy())
        np.testing.assert_array_equal(q[g].cpu().numpy(), rq)
        np.testing.assert_array_equal(sf[g].cpu().numpy(), np.repeat(rs, 128, axis=1))
        np.testing.assert_array_equal(sd[g].cpu().numpy(), np.repeat(rs.T, 128, axis=1))


@pytest.mark.parametrize("M,G,K", [(700, 5, 256), (3000, 64, 128), (128, 1, 7168)])
def test_quant_token_tiles_bit_exact(gpu, M, G, K):
    x = _bf16_data((M, K), 3)
    off = inputs.random_segments(M, G, 5, empty_frac=0.25, skew=0.5)
    ldm = abi.moe_padded_rows_bound(M, G, 128)
    poff = torch.empty(G + 1, dtype=torch.int64, device=DEV)
    abi.moe_padded_offsets(off.to(DEV), M, poff)
    qT = torch.full((K, ldm), 0xAA, dtype=torch.uint8, device=DEV)
    s = torch.empty((ldm // 128, K), dtype=torch.float32, device=DEV)
    abi.moe_quant_fp8_token_tiles(x.to(DEV), off.to(DEV), poff, qT, s)
    rq, rs, rpoff = fp8.quantize_token_tiles(x.float().numpy(), off.numpy())
    np.testing.assert_array_equal(poff.cpu().numpy(), rpoff)
    mp = int(rpoff[-1])
    np.testing.assert_array_equal(qT.cpu().numpy()[:, :mp].T, rq)
    np.testing.assert_array_equal(s.cpu().numpy()[:mp // 128], rs)


def _oracle_weights(W):
    """Oracle block codes of W [G, K, N] (one layout, W's own, for both GEMMs)
    and the block scale expanded along each GEMM's output columns."""
    qs = [fp8.quantize_blocks(W[g].float().numpy()) for g in range(W.shape[0])]
    deq = np.stack([fp8.dequantize_blocks(q, s) for q, s in qs])
    q = torch.from_numpy(np.stack([q for q, _ in qs]).copy())
    sf = torch.from_numpy(np.stack([np.repeat(s, 128, axis=1) for _, s in qs]).copy())
    sd = torch.from_numpy(np.stack([np.repeat(s.T, 128, axis=1) for _, s in qs]).copy())
    return deq, q, sf, sd


def _oracle_rows(A):
    q, s = fp8.quantize_rows(A.float().numpy())
    return fp8.dequantize_rows(q, s), torch.from_numpy(q), torch.from_numpy(s.T.copy())


@pytest.mark.parametrize("M,G,K,N,swiglu", [(1000, 5, 256, 384, False), (2600, 8, 512, 512, True),
                                             (129, 1, 128, 256, True), (700, 3, 256, 384, True)])
def test_fp8_grouped_gemm_fwd_dgrad(gpu, M, G, K, N, swiglu):
    print(f"fp8 gemm M={M} G={G} K={K} N={N} swiglu={swiglu}", flush=True)
    off = inputs.random_segments(M, G, 7, empty_frac=0.2)
    o = off.numpy()
    A = _bf16_data((M, K), 8)
    W = (_bf16_data((G, K, N), 9) * K ** -0.5)
    Ad, Aq, As = _oracle_rows(A)
    Wd, qw, sf, sd = _oracle_weights(W)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    H = torch.empty((M, N // 2), dtype=torch.bfloat16, device=DEV) if swiglu else None
    abi.moe_grouped_gemm_fp8_fwd(Aq.to(DEV), As.to(DEV), qw.to(DEV), sf.to(DEV), off.to(DEV), C, H,
                                 epilogue=abi.EPI_SWIGLU if swiglu else abi.EPI_NONE)
    ref = oracle.grouped_gemm_fwd(Ad, Wd, o)
    assert_close("C", C, ref, TOL["fp8"])
    assert rel_small(C, ref)
    if swiglu:
        assert_close("H", H, oracle.swiglu(ref), TOL["fp8"])
    # dgrad: dA [M, K] = dC [M, N] . W^T, dC quantized along N
    dC = _bf16_data((M, N), 10)
    dCd, dCq, dCs = _oracle_rows(dC)
    dA = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    abi.moe_grouped_gemm_fp8_dgrad(dCq.to(DEV), dCs.to(DEV), qw.to(DEV), sd.to(DEV), off.to(DEV), dA)
    refd = oracle.grouped_gemm_dgrad(dCd, Wd, o)
    assert_close("dA", dA, refd, TOL["fp8"])
    assert rel_small(dA, refd)


def rel_small(got, ref):
    from gpu_util import rel_err
    return rel_err(got, ref) < 1e-2


@pytest.mark.parametrize("M,G,K,N", [(1500, 6, 256, 384), (1500, 6, 256, 512), (300, 1, 128, 128)])
def test_fp8_grouped_gemm_wgrad(gpu, M, G, K, N):
    off = inputs.random_segments(M, G, 11, empty_frac=0.3, skew=0.5)
    A = _bf16_data((M, K), 12)
    dC = _bf16_data((M, N), 13)
    qa, sa, poff = fp8.quantize_token_tiles(A.float().numpy(), off.numpy())
    qc, sc, _ = fp8.quantize_token_tiles(dC.float().numpy(), off.numpy())
    ldm = abi.moe_padded_rows_bound(M, G, 128)
    mp = int(poff[-1])
    At = torch.zeros((K, ldm), dtype=torch.uint8)
    At[:, :mp] = torch.from_numpy(qa.T.copy())
    Ct = torch.zeros((N, ldm), dtype=torch.uint8)
    Ct[:, :mp] = torch.from_numpy(qc.T.copy())
    Sa = torch.ones((ldm // 128, K), dtype=torch.float32)
    Sa[:mp // 128] = torch.from_numpy(sa)
    Sc = torch.ones((ldm // 128, N), dtype=torch.float32)
    Sc[:mp // 128] = torch.from_numpy(sc)
    ref = oracle.grouped_gemm_wgrad(fp8.dequantize_token_tiles(qa, sa),
                                    fp8.dequantize_token_tiles(qc, sc), poff)
    for dt in (torch.bfloat16, torch.float32):
        dB = torch.full((G, K, N), float("nan"), dtype=dt, device=DEV)
        abi.moe_grouped_gemm_fp8_wgrad(At.to(DEV), Sa.to(DEV), Ct.to(DEV), Sc.to(DEV),
                                       torch.from_numpy(poff).to(DEV), dB)
        assert_close(f"dB {dt}", dB, ref, TOL["fp8"])
        assert rel_small(dB, ref)


SMALL_FP8 = inputs.LayerConfig("small_fp8_shared", T=400, d=256, E=8, k=2, f=256, fs=128,
                               gemm="fp8", score="sigmoid", bias="normal")


@pytest.mark.parametrize("cfg", [SMALL_FP8,
                                 dataclasses.replace(SMALL_FP8, name="small_fp8_capacity",
                                                     capacity_factor=0.8, bias="zipf"),
                                 dataclasses.replace(SMALL_FP8, name="small_fp8_softmax", fs=0,
                                                     score="softmax", bias="none", k=4)],
                         ids=lambda c: c.name)
def test_layer_fp8(gpu, cfg):
    print(f"fp8 layer {cfg.name}", flush=True)
    inp = inputs.layer_inputs(cfg, 0)
    w = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer = MoELayer(cfg, w, DEV)
    layer.forward(w["x"])
    layer.backward(w["dout"])
    torch.cuda.synchronize()
    shared = (np64(inp["ws13"]), np64(inp["ws2"])) if cfg.fs else None
    bias = None if inp["logit_bias"] is None else inp["logit_bias"].numpy()
    ref = fp8.layer_fp8(np64(inp["x"]), inp["w_r"].numpy(), np64(inp["w13"]), np64(inp["w2"]),
                        np64(inp["dout"]), cfg.k, cfg.score, cfg.renorm, logit_bias=bias,
                        shared=shared, z=layer.logits.cpu().numpy(),
                        capacity=(oracle.capacity_of(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
                                  if cfg.capacity_factor else None))
    if cfg.capacity_factor:
        assert (layer.dst_row < 0).sum() > 0  # some pairs are dropped
    assert_close("logits (oracle's own)", layer.logits,
                 oracle.router_logits(np64(inp["x"]), inp["w_r"].numpy(), bias), TOL["f32"])
    r = ref["route"]
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), r["dst_row"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), r["offsets"])
    assert_close("out", layer.out, ref["out"], TOL["fp8"])
    g = layer.grads()
    for name in ["dx", "d_logits", "dW_r", "dW13", "dW2"] + (["dWs13", "dWs2"] if cfg.fs else []):
        assert_close(name, g[name], ref[name], TOL["fp8"])


def _bf16_neighbours(v):
    """The bf16 values just below and just above each of v (positive, finite)."""
    b = torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    u = b.view(torch.int16).to(torch.int32)
    lo = (u - 1).to(torch.int16).view(torch.bfloat16)
    hi = (u + 1).to(torch.int16).view(torch.bfloat16)
    return lo.float().numpy(), hi.float().numpy()


def _e4m3_sweep(limit):
    """bf16 values probing every rounding decision of E4M3 up to ``limit``:
    all finite E4M3 magnitudes, every midpoint between neighbours (including
    the subnormal ones and the one between 0 and the least subnormal), the
    bf16 neighbours of each, far-underflowing values, and both signs."""
    vals = np.unique(np.abs(fp8.decode(np.arange(0x7F))))            # 0 .. 448
    mids = (vals[1:] + vals[:-1]) / 2
    pts = np.concatenate([vals, mids])
    pts = pts[pts > 0]
    lo, hi = _bf16_neighbours(pts)
    extra = [2.0 ** -20, 2.0 ** -126, 2.0 ** -133, 0.0]
    pos = np.concatenate([pts, lo, hi, extra])
    pos = pos[(pos >= 0) & (pos <= limit)]
    v = np.concatenate([pos, -pos]).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).float().numpy()   # exactly bf16 values


def test_e4m3_dense_sweep_rows(gpu):
    """The hardware E4M3 conversion in moe_quant_fp8_rows against the
    definition encoder, bit for bit, at unit scale: every 128-tile carries
    448 (so scale = inv = 1 exactly and each code is encode(v) itself) and
    127 values of the sweep (midpoints with ties to even, their bf16
    neighbours, subnormal midpoints, +-0, underflow)."""
    v = _e4m3_sweep(448.0)
    n_tiles = (len(v) + 126) // 127
    x = np.zeros((n_tiles, 128), np.float32)
    x[:, 0] = 448.0
    x.reshape(-1)[np.concatenate([np.arange(1 + 128 * i, 128 * (i + 1)) for i in range(n_tiles)])[:len(v)]] = v
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(xb.float(), torch.from_numpy(x))
    q = torch.empty((n_tiles, 128), dtype=torch.uint8, device=DEV)
    sT = torch.empty((1, n_tiles), dtype=torch.float32, device=DEV)
    abi.moe_quant_fp8_rows(xb.to(DEV), q, sT)
    assert (sT.cpu().numpy() == 1.0).all()
    got = q.cpu().numpy()
    np.testing.assert_array_equal(got, fp8.encode(x))
    assert len(v) > 1000


def test_e4m3_dense_sweep_mx_rows(gpu):
    """The same sweep through moe_quant_mxfp8_rows at shared exponent 0: every
    32-block carries 256 (X = floor(log2 256) - 8 = 0, an exact scaling by 1),
    so the codes are encode(v); here the sweep also spans the saturating band
    [448, 512) (bf16 values 448, 450, ..., 510 -> 448)."""
    band = np.arange(448.0, 512.0, 2.0)
    v = np.concatenate([_e4m3_sweep(448.0), band, -band]).astype(np.float32)
    n_blk = (len(v) + 30) // 31
    x = np.zeros((n_blk, 32), np.float32)
    x[:, 0] = 256.0
    flat = np.concatenate([np.arange(1 + 32 * i, 32 * (i + 1)) for i in range(n_blk)])[:len(v)]
    x.reshape(-1)[flat] = v
    pad = (-x.size) % 128                      # rows of K = 128 (4 blocks each)
    xr = np.concatenate([x.reshape(-1), np.tile(np.array([256.0] + [0.0] * 31, np.float32),
                                                 pad // 32)]).reshape(-1, 128)
    xb = torch.from_numpy(xr).to(torch.bfloat16)
    assert torch.equal(xb.float(), torch.from_numpy(xr))
    M = xr.shape[0]
    q = torch.empty((M, 128), dtype=torch.uint8, device=DEV)
    s = torch.empty((M, 4), dtype=torch.uint8, device=DEV)
    abi.moe_quant_mxfp8_rows(xb.to(DEV), q, s)
    assert (s.cpu().numpy() == 127).all()
    np.testing.assert_array_equal(q.cpu().numpy(), fp8.encode(xr))
