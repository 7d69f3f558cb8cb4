"""Pins of the oracle's whole-layer forward and backward:
  * brute-force dense evaluation (every token through every expert, gated by
    a dense [T, E] weight matrix) against the per-token loop;
  * the per-op chain permute -> grouped GEMM -> SwiGLU -> grouped GEMM ->
    combine against the per-token loop;
  * reductions to a dense SwiGLU FFN (E = 1, k = 1; all experts identical);
  * central finite differences of every gradient, for all four score modes;
  * the permute -> unpermute round trip giving k * x.
"""
import numpy as np
import pytest

import oracle


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _dense_ffn(x, w13, w2):
    f = w13.shape[1] // 2
    return (_silu(x @ w13[:, :f]) * (x @ w13[:, f:])) @ w2


def _make(seed, T=16, d=12, E=4, k=2, f=10, fs=0, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, E)) / np.sqrt(d)
    w13 = rng.standard_normal((E, d, 2 * f)) / np.sqrt(d)
    w2 = rng.standard_normal((E, f, d)) / np.sqrt(f)
    b = rng.standard_normal(E).astype(np.float32) * 0.7 if bias else None
    shared = None
    if fs:
        shared = (rng.standard_normal((d, 2 * fs)) / np.sqrt(d), rng.standard_normal((fs, d)) / np.sqrt(fs))
    dout = rng.standard_normal((T, d))
    return x, w_r, w13, w2, b, shared, dout


MODES = [(oracle.SOFTMAX, True), (oracle.SOFTMAX, False), (oracle.SIGMOID, True), (oracle.SIGMOID, False)]


@pytest.mark.parametrize("score,renorm", MODES)
def test_dense_brute_force(score, renorm):
    x, w_r, w13, w2, b, shared, _ = _make(1, fs=6, bias=True)
    T, E, k = x.shape[0], w13.shape[0], 2
    c = oracle.layer_forward(x, w_r, w13, w2, k, score, renorm, logit_bias=b, shared=shared)
    G = np.zeros((T, E))
    np.put_along_axis(G, c["route"]["topk_idx"].astype(int), c["route"]["topk_w"], axis=1)
    dense = sum(G[:, e:e + 1] * _dense_ffn(x, w13[e], w2[e]) for e in range(E))
    dense = dense + _dense_ffn(x, *shared)
    np.testing.assert_allclose(c["out"], dense, rtol=0, atol=1e-12)


def test_op_chain_matches_per_token_loop():
    x, w_r, w13, w2, b, shared, dout = _make(2, T=23, E=5, k=3, fs=4, bias=True)
    k = 3
    c = oracle.layer_forward(x, w_r, w13, w2, k, oracle.SOFTMAX, True, logit_bias=b, shared=shared)
    r = c["route"]
    xp = oracle.permute(x, r["src_token"])
    ab = oracle.grouped_gemm_fwd(xp, w13, r["offsets"])
    h = oracle.swiglu(ab)
    y = oracle.grouped_gemm_fwd(h, w2, r["offsets"])
    ys = _dense_ffn(x, *shared)
    out = oracle.unpermute_combine(y, r["topk_w"], r["dst_row"], ys)
    np.testing.assert_allclose(out, c["out"], rtol=0, atol=1e-12)
    # backward through the same chain
    g = oracle.layer_backward(c, dout)
    dy, dw = oracle.unpermute_combine_bwd(dout, y, r["topk_w"], r["dst_row"])
    np.testing.assert_allclose(dw, g["d_topk_w"], rtol=0, atol=1e-12)
    dh = oracle.grouped_gemm_dgrad(dy, w2, r["offsets"])
    dW2 = oracle.grouped_gemm_wgrad(h, dy, r["offsets"])
    np.testing.assert_allclose(dW2, g["dW2"], rtol=0, atol=1e-12)
    dab = oracle.swiglu_bwd(dh, ab)
    dxp = oracle.grouped_gemm_dgrad(dab, w13, r["offsets"])
    dW13 = oracle.grouped_gemm_wgrad(xp, dab, r["offsets"])
    np.testing.assert_allclose(dW13, g["dW13"], rtol=0, atol=1e-12)
    dz = oracle.route_bwd(c["z"], r["topk_idx"], r["topk_w"], dw, oracle.SOFTMAX, True)
    dWr, dxr = oracle.router_logits_bwd(x, w_r, dz)
    np.testing.assert_allclose(dWr, g["dW_r"], rtol=0, atol=1e-12)
    # shared expert backward, written densely
    ws13, ws2 = shared
    fs = ws2.shape[0]
    a, bb = x @ ws13[:, :fs], x @ ws13[:, fs:]
    s = 1 / (1 + np.exp(-a))
    dhs = dout @ ws2.T
    dabs = np.concatenate([dhs * bb * s * (1 + a * (1 - s)), dhs * a * s], 1)
    dx = oracle.permute_bwd(dxp, r["dst_row"], addends=(dabs @ ws13.T, dxr))
    np.testing.assert_allclose(dx, g["dx"], rtol=0, atol=1e-12)


def test_single_expert_is_dense_ffn():
    x, w_r, w13, w2, _, _, dout = _make(3, E=1)
    c = oracle.layer_forward(x, w_r, w13, w2, 1, oracle.SOFTMAX, True)
    np.testing.assert_allclose(c["route"]["topk_w"], 1.0)
    np.testing.assert_allclose(c["out"], _dense_ffn(x, w13[0], w2[0]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
def test_identical_experts_reduce_to_dense(score):
    """Renormalised weights sum to one, so with identical experts the layer is
    the dense FFN for any routing, sum_e dW_e is the dense dW, and the router
    gets no gradient."""
    x, w_r, w13, w2, b, _, dout = _make(4, E=6, k=3, bias=True)
    w13[:] = w13[0]
    w2[:] = w2[0]
    c = oracle.layer_forward(x, w_r, w13, w2, 3, score, True, logit_bias=b)
    np.testing.assert_allclose(c["out"], _dense_ffn(x, w13[0], w2[0]), rtol=0, atol=1e-12)
    g = oracle.layer_backward(c, dout)
    # dense backward by hand
    f = w13.shape[2] // 2
    a, bb = x @ w13[0][:, :f], x @ w13[0][:, f:]
    s = 1 / (1 + np.exp(-a))
    h = a * s * bb
    dh = dout @ w2[0].T
    dab = np.concatenate([dh * bb * s * (1 + a * (1 - s)), dh * a * s], 1)
    np.testing.assert_allclose(g["dW13"].sum(0), x.T @ dab, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dW2"].sum(0), h.T @ dout, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dx"], dab @ w13[0].T, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dW_r"], 0.0, atol=1e-12)


def _gap_ok(z, k, margin):
    s = np.sort(z, axis=1)[:, ::-1]
    return np.all(s[:, k - 1] - s[:, k] > margin)


@pytest.mark.parametrize("score,renorm", MODES)
def test_backward_finite_differences(score, renorm):
    """Every gradient of L = sum(out * dout) against central differences of
    the forward, with the selection held fixed (keys well separated)."""
    for seed in range(100):
        x, w_r, w13, w2, b, shared, dout = _make(seed, T=6, d=5, E=4, k=2, f=3, fs=2, bias=True)
        z = x @ w_r + b
        if _gap_ok(z, 2, 1e-2):
            break
    k = 2
    c = oracle.layer_forward(x, w_r, w13, w2, k, score, renorm, logit_bias=b, shared=shared,
                             z=(x @ w_r + b))
    g = oracle.layer_backward(c, dout)
    idx = c["route"]["topk_idx"]

    def loss(x_, w_r_, w13_, w2_, ws13_, ws2_):
        zz = x_ @ w_r_ + b            # float64 keys, selection fixed
        w = oracle.gates(zz, idx, score, renorm)
        out = np.zeros_like(x_)
        for t in range(x_.shape[0]):
            for j in range(k):
                e = idx[t, j]
                out[t] += w[t, j] * _dense_ffn(x_[t:t + 1], w13_[e], w2_[e])[0]
        out += _dense_ffn(x_, ws13_, ws2_)
        return (out * dout).sum()

    args = [x, w_r, w13, w2, shared[0], shared[1]]
    names = ["dx", "dW_r", "dW13", "dW2", "dWs13", "dWs2"]
    eps = 1e-6
    for i, name in enumerate(names):
        arr = args[i]
        num = np.zeros_like(arr)
        for pos in np.ndindex(arr.shape):
            keep = arr[pos]
            arr[pos] = keep + eps
            lp = loss(*args)
            arr[pos] = keep - eps
            lm = loss(*args)
            arr[pos] = keep
            num[pos] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=0, atol=2e-7, err_msg=name)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_round_trip_is_k_times_x(k):
    rng = np.random.default_rng(9)
    T, E, d = 33, 6, 8
    x = rng.integers(-512, 512, size=(T, d)) / 256.0
    z = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(z, k, oracle.SOFTMAX, True)
    xp = oracle.permute(x, r["src_token"])
    back = oracle.unpermute_combine(xp, np.ones((T, k)), r["dst_row"])
    np.testing.assert_array_equal(back, k * x)
    np.testing.assert_array_equal(oracle.permute_bwd(xp, r["dst_row"]), k * x)


def test_expert_wgrad_columns_match_full_backward():
    x, w_r, w13, w2, b, _, dout = _make(6, T=20, E=3, k=2)
    c = oracle.layer_forward(x, w_r, w13, w2, 2, oracle.SOFTMAX, True)
    g = oracle.layer_backward(c, dout)
    r = c["route"]
    f = w13.shape[2] // 2
    cols = np.array([0, 3, f - 1])
    for e in range(3):
        ts, js = np.nonzero(r["topk_idx"] == e)
        dy = r["topk_w"][ts, js][:, None] * dout[ts]
        d1, d3, d2 = oracle.expert_wgrad_columns(x[ts], dy, w13[e], w2[e], cols)
        np.testing.assert_allclose(d1, g["dW13"][e][:, cols], rtol=0, atol=1e-12)
        np.testing.assert_allclose(d3, g["dW13"][e][:, f + cols], rtol=0, atol=1e-12)
        np.testing.assert_allclose(d2, g["dW2"][e][cols, :], rtol=0, atol=1e-12)


@pytest.mark.parametrize("score,renorm", MODES)
def test_gated_arrangement_equals_baseline(score, renorm):
    """The memory-saving arrangement (routing weight applied before W2, an
    unweighted combine, the weight gradient taken over the ffn axis) computes
    the same output and gradients as the baseline, by linearity: agreement to
    fp64 rounding, with routing replayed and with a shared expert."""
    x, w_r, w13, w2, b, shared, dout = _make(21, T=20, d=12, E=5, k=2, f=7, fs=4, bias=True)
    for given in (None, np.stack([np.array([t % 5, (t + 2) % 5]) for t in range(20)])):
        c0 = oracle.layer_forward(x, w_r, w13, w2, 2, score, renorm, logit_bias=b, shared=shared,
                                  given_experts=given)
        c1 = oracle.layer_forward_gated(x, w_r, w13, w2, 2, score, renorm, logit_bias=b,
                                        shared=shared, given_experts=given)
        np.testing.assert_allclose(c1["out"], c0["out"], rtol=0, atol=1e-12)
        g0 = oracle.layer_backward(c0, dout)
        g1 = oracle.layer_backward_gated(c1, dout)
        for name in ["dx", "d_logits", "dW_r", "dW13", "dW2", "d_topk_w", "dWs13", "dWs2"]:
            np.testing.assert_allclose(g1[name], g0[name], rtol=0, atol=1e-11, err_msg=name)
