"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (MoELayer forward + backward on GPU-resident inputs).

Routing, counts, offsets and the permutation are compared in full and
bit-exactly (inputs are drawn with no near-tie at the top-k boundary).  The
oracle then recomputes, one by one, the output, dx and router gradient of a
sample of tokens (including tokens of the largest, a median and the smallest
non-empty expert), and full columns of dW1 / dW3 and rows of dW2 of a sample
of experts; each compared by max|err| / max|ref| within the bf16 bound."""
import numpy as np
import pytest
import torch

import oracle
from routing_grouped_gemm_router_amd import inputs
from routing_grouped_gemm_router_amd.layer import MoELayer
from gpu_util import TOL, assert_close, near_tie_tokens, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs_without_near_ties(cfg, seed, rel_gap=1e-4, attempts=10):
    inp = inputs.layer_inputs(cfg, seed, DEV)
    w_r = inp["w_r"].cpu().numpy()
    bias = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    for attempt in range(attempts):
        z = oracle.router_logits(np64(inp["x"]), w_r, bias)
        bad = near_tie_tokens(z, cfg.k, rel_gap)
        if len(bad) == 0:
            return inp, z
        print(f"  resampling {len(bad)} near-tie token rows", flush=True)
        inputs.resample_rows(inp["x"], [int(t) for t in bad], seed, attempt)
    raise RuntimeError("could not draw inputs without near-ties")


def _sample_tokens(r, n_random, seed):
    counts = r["counts"]
    nz = np.nonzero(counts)[0]
    big, small = nz[np.argmax(counts[nz])], nz[np.argmin(counts[nz])]
    med = nz[np.argsort(counts[nz])[len(nz) // 2]]
    toks = set()
    for e in (big, med, small):
        seg = r["src_token"][r["offsets"][e]:r["offsets"][e + 1]]
        toks.update(int(t) for t in seg[:1])
    rng = np.random.default_rng(seed)
    T = r["topk_idx"].shape[0]
    toks.update(int(t) for t in rng.choice(T, n_random, replace=False))
    toks.add(T - 1)
    return sorted(toks), [int(big), int(med), int(small)]


@pytest.mark.parametrize("name,n_tok,n_exp_rand", [
    ("llama3_8b_e8k2", 5, 1),
    ("qwen3_235b_e128k8", 5, 1),
    ("deepseek_v3_e256k8", 4, 1),
])
def test_fullsize_layer(gpu, name, n_tok, n_exp_rand):
    cfg = inputs.CONFIGS[name]
    print(f"full-size layer {name}", flush=True)
    inp, z = _inputs_without_near_ties(cfg, seed=0)
    layer = MoELayer(cfg, inp, DEV)
    layer.forward(inp["x"])
    layer.backward(inp["dout"])
    torch.cuda.synchronize()

    # ---- routing, in full and bit-exact
    assert_close("logits", layer.logits, z, TOL["f32"])
    r = oracle.route(z, cfg.k, cfg.score, cfg.renorm)
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), r["topk_idx"])
    np.testing.assert_array_equal(layer.counts.cpu().numpy(), r["counts"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), r["offsets"])
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), r["dst_row"])
    np.testing.assert_array_equal(layer.src_token.cpu().numpy(), r["src_token"])
    assert_close("topk_w", layer.topk_w, r["topk_w"], TOL["f32"])

    tol = TOL[cfg.gemm]
    toks, experts = _sample_tokens(r, n_tok, seed=1)
    print(f"  sampled tokens {toks}; experts {experts}", flush=True)
    w_r = inp["w_r"].cpu().numpy().astype(np.float64)
    shared = None
    if cfg.fs:
        shared = (np64(inp["ws13"]), np64(inp["ws2"]))
    cache = {}

    def expert(e):
        if e not in cache:
            cache.clear() if len(cache) > 8 else None
            cache[e] = (np64(inp["w13"][e]), np64(inp["w2"][e]))
        return cache[e]

    # ---- per-token outputs, dx and router gradient
    out_ref, dx_ref, dz_ref = [], [], []
    for t in toks:
        x_t = np64(inp["x"][t])
        dout_t = np64(inp["dout"][t])
        o = np.zeros(cfg.d)
        dx = np.zeros(cfg.d)
        dw = np.zeros((1, cfg.k))
        for j in range(cfg.k):
            e = int(r["topk_idx"][t, j])
            w13e, w2e = expert(e)
            a, b, h, y = oracle.expert_ffn(x_t, w13e, w2e)
            o += r["topk_w"][t, j] * y
            dw[0, j] = dout_t @ y
            dxe, _, _ = oracle.expert_ffn_bwd(x_t, w13e, w2e, a, b, h, r["topk_w"][t, j] * dout_t)
            dx += dxe
        if shared is not None:
            a, b, h, y = oracle.expert_ffn(x_t, *shared)
            o += y
            dxs, _, _ = oracle.expert_ffn_bwd(x_t, shared[0], shared[1], a, b, h, dout_t)
            dx += dxs
        dz = oracle.route_bwd(z[t:t + 1], r["topk_idx"][t:t + 1], r["topk_w"][t:t + 1], dw,
                              cfg.score, cfg.renorm)
        dx += (dz @ w_r.T)[0]
        out_ref.append(o)
        dx_ref.append(dx)
        dz_ref.append(dz[0])
    idx = torch.tensor(toks, device=DEV)
    assert_close("out (sampled tokens)", layer.out[idx], np.stack(out_ref), tol)
    assert_close("dx (sampled tokens)", layer.dx[idx], np.stack(dx_ref), tol)
    assert_close("d_logits (sampled tokens)", layer.d_logits[idx], np.stack(dz_ref), tol)

    # ---- weight gradients: whole columns / rows of sampled experts
    rng = np.random.default_rng(2)
    nz = np.nonzero(r["counts"])[0]
    exps = experts + [int(e) for e in rng.choice(nz, n_exp_rand, replace=False)]
    cols = np.unique(np.concatenate([[0, cfg.f - 1], rng.choice(cfg.f, 14, replace=False)]))
    x_all = None
    for e in exps:
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        toks_e = r["src_token"][lo:hi].astype(np.int64)
        slots = np.array([int(np.nonzero(r["topk_idx"][t] == e)[0][0]) for t in toks_e])
        x_rows = np64(inp["x"][torch.from_numpy(toks_e).to(DEV)])
        dout_rows = np64(inp["dout"][torch.from_numpy(toks_e).to(DEV)])
        dy_rows = r["topk_w"][toks_e, slots][:, None] * dout_rows
        w13e, w2e = expert(e)
        d1, d3, d2 = oracle.expert_wgrad_columns(x_rows, dy_rows, w13e, w2e, cols)
        c = torch.from_numpy(cols).to(DEV)
        assert_close(f"dW1[{e}] cols ({hi - lo} rows)", layer.dw13[e][:, c], d1, tol)
        assert_close(f"dW3[{e}] cols", layer.dw13[e][:, cfg.f + c], d3, tol)
        assert_close(f"dW2[{e}] rows", layer.dw2[e][c, :], d2, tol)
    if shared is not None:
        x_all = np64(inp["x"])
        d1, d3, d2 = oracle.expert_wgrad_columns(x_all, np64(inp["dout"]), shared[0], shared[1],
                                                 cols)
        c = torch.from_numpy(cols).to(DEV)
        assert_close("dWs1 cols", layer.dws13[0][:, c], d1, tol)
        assert_close("dWs3 cols", layer.dws13[0][:, cfg.fs + c], d3, tol)
        assert_close("dWs2 rows", layer.dws2[0][c, :], d2, tol)
    del layer, inp
    torch.cuda.empty_cache()


def test_fullsize_fp8_layer(gpu):
    """The blockwise-fp8 DeepSeek-V3 layer at its full size (T = 32768), in
    the launch configuration bench.py times.  Routing in full and bit-exact;
    then the oracle's quantize-at-every-GEMM-input chain (oracle.fp8, the
    blockwise recipe) recomputed one token at a time -- 1 x 128 activation
    tiles are row-local, and each involved expert's weights are quantized in
    128 x 128 blocks -- for the output and dx of a sampled token; and, for
    the smallest non-empty expert, its whole segment quantized in 128-token
    tiles for columns of dW1 / dW3 and rows of dW2.  Within the fp8 bound."""
    from oracle import fp8

    cfg = inputs.CONFIGS["deepseek_v3_fp8"]
    print("full-size fp8 layer", flush=True)
    inp, z = _inputs_without_near_ties(cfg, seed=0)
    layer = MoELayer(cfg, inp, DEV)
    layer.forward(inp["x"])
    layer.backward(inp["dout"])
    torch.cuda.synchronize()
    r = oracle.route(z, cfg.k, cfg.score, cfg.renorm)
    for name in ("topk_idx", "counts", "offsets", "dst_row", "src_token"):
        np.testing.assert_array_equal(getattr(layer, name).cpu().numpy(), r[name], err_msg=name)
    tol = TOL["fp8"]

    def q_rows(a):  # bf16 storage, then 1 x 128 tiles
        q, s = fp8.quantize_rows(fp8.to_bf16(np.atleast_2d(a)))
        return fp8.dequantize_rows(q, s)

    def q_weight(w):  # 128 x 128 blocks (the same blocks serve the forward and dgrad)
        q, s = fp8.quantize_blocks(fp8.to_bf16(w))
        return fp8.dequantize_blocks(q, s)

    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = (q_weight(np64(inp["w13"][e])), q_weight(np64(inp["w2"][e])))
        return cache[e]

    def chain(x_rows, dy_rows, w13q, w2q):
        """Forward and data gradient of one expert on rows (oracle.fp8's chain)."""
        ab = q_rows(x_rows) @ w13q
        h = oracle.swiglu(ab)
        y = q_rows(h) @ w2q
        dh = q_rows(dy_rows) @ w2q.T
        dab = oracle.swiglu_bwd(dh, ab)
        dx = q_rows(dab) @ w13q.T
        return h, y, dab, dx

    counts = r["counts"]
    nz = np.nonzero(counts)[0]
    med = nz[np.argsort(counts[nz])[len(nz) // 2]]
    t = int(r["src_token"][r["offsets"][med]])
    print(f"  sampled token {t}", flush=True)
    x_t, dout_t = np64(inp["x"][t])[None], np64(inp["dout"][t])[None]
    o = np.zeros((1, cfg.d))
    dx = np.zeros((1, cfg.d))
    dw = np.zeros((1, cfg.k))
    for j in range(cfg.k):
        e = int(r["topk_idx"][t, j])
        w13q, w2q = expert(e)
        _, y, _, _ = chain(x_t, np.zeros((1, cfg.d)), w13q, w2q)
        dw[0, j] = (dout_t @ y.T)[0, 0]
        _, y, _, dxe = chain(x_t, fp8.to_bf16(r["topk_w"][t, j] * dout_t), w13q, w2q)
        o += r["topk_w"][t, j] * y
        dx += dxe
    ws = (q_weight(np64(inp["ws13"])), q_weight(np64(inp["ws2"])))
    _, ys, _, dxs = chain(x_t, dout_t, *ws)
    o += ys
    dx += dxs
    dz = oracle.route_bwd(z[t:t + 1], r["topk_idx"][t:t + 1], r["topk_w"][t:t + 1], dw, cfg.score,
                          cfg.renorm)
    dx += dz @ inp["w_r"].cpu().numpy().astype(np.float64).T
    assert_close("out (sampled token)", layer.out[t:t + 1], o, tol)
    assert_close("dx (sampled token)", layer.dx[t:t + 1], dx, tol)
    assert_close("d_logits (sampled token)", layer.d_logits[t:t + 1], dz, tol)

    # weight gradients of the smallest non-empty expert, whole segment
    e = int(nz[np.argmin(counts[nz])])
    lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
    toks_e = r["src_token"][lo:hi].astype(np.int64)
    slots = np.array([int(np.nonzero(r["topk_idx"][u] == e)[0][0]) for u in toks_e])
    x_rows = np64(inp["x"][torch.from_numpy(toks_e).to(DEV)])
    dy_rows = fp8.to_bf16(r["topk_w"][toks_e, slots][:, None]
                          * np64(inp["dout"][torch.from_numpy(toks_e).to(DEV)]))
    w13q, w2q = expert(e)
    h, _, dab, _ = chain(x_rows, dy_rows, w13q, w2q)
    seg = np.array([0, hi - lo])

    def tiles(a):
        q, s, _ = fp8.quantize_token_tiles(fp8.to_bf16(a), seg)
        return fp8.dequantize_token_tiles(q, s)

    rng = np.random.default_rng(2)
    cols = np.unique(np.concatenate([[0, cfg.f - 1], rng.choice(cfg.f, 14, replace=False)]))
    xt, dabt, ht, dyt = tiles(x_rows), tiles(dab), tiles(h), tiles(dy_rows)
    c = torch.from_numpy(cols).to(DEV)
    print(f"  expert {e}: {hi - lo} rows", flush=True)
    assert_close(f"dW1[{e}] cols", layer.dw13[e][:, c], xt.T @ dabt[:, cols], tol)
    assert_close(f"dW3[{e}] cols", layer.dw13[e][:, cfg.f + c], xt.T @ dabt[:, cfg.f + cols], tol)
    assert_close(f"dW2[{e}] rows", layer.dw2[e][c, :], ht[:, cols].T @ dyt, tol)
    del layer, inp
    torch.cuda.empty_cache()
