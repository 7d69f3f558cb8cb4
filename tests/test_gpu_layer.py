"""Whole-layer parity, forward and backward, of the HIP path (MoELayer, all
C-ABI calls in sequence) against the oracle's per-token loop on the same
seeded inputs.  The oracle's own fp32 logits are compared with the GPU's
(1e-5 of max|ref|); the oracle then routes from the GPU's logits tensor, so
routing is compared bit-exactly with no re-drawn inputs, and every output
and gradient by max|err|/max|ref|."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from routing_grouped_gemm_router_amd import inputs
from routing_grouped_gemm_router_amd.layer import MoELayer
from gpu_util import TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL_BF16 = inputs.LayerConfig("small_bf16_shared", T=300, d=256, E=8, k=2, f=256, fs=128,
                                score="sigmoid", bias="normal")
SMALL_BF16_SOFTMAX = inputs.LayerConfig("small_bf16_zipf", T=513, d=128, E=16, k=4, f=128,
                                        bias="zipf")


def _run(cfg, seed, recompute_act=False, gate_in_ffn=False):
    print(f"layer {cfg.name} seed={seed} recompute={recompute_act} gated={gate_in_ffn}",
          flush=True)
    inp = inputs.layer_inputs(cfg, seed)
    w = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer = MoELayer(cfg, w, DEV, recompute_act=recompute_act, gate_in_ffn=gate_in_ffn)
    layer.forward(w["x"])
    layer.backward(w["dout"])
    torch.cuda.synchronize()
    shared = (np64(inp["ws13"]), np64(inp["ws2"])) if cfg.fs else None
    bias = None if inp["logit_bias"] is None else inp["logit_bias"].numpy()
    given = inp["topk_idx_in"].numpy() if cfg.routing == "balanced" else None
    z_own = oracle.router_logits(np64(inp["x"]), inp["w_r"].numpy(), bias)
    z = layer.logits.cpu().numpy()  # the oracle routes from the GPU's fp32 logits
    if cfg.expert_bias_std > 0:
        # the experts chosen on the biased keys; the oracle layer then takes
        # the routing weights from the unbiased scores, as the route does
        given = oracle.route_expert_bias(z, inp["expert_bias"].numpy(), cfg.k,
                                         cfg.renorm)["topk_idx"]
    fwd = oracle.layer_forward_gated if gate_in_ffn else oracle.layer_forward
    bwd = oracle.layer_backward_gated if gate_in_ffn else oracle.layer_backward
    cap = (oracle.capacity_of(cfg.capacity_factor, cfg.T, cfg.k, cfg.E)
           if cfg.capacity_factor > 0 else None)
    c = fwd(np64(inp["x"]), inp["w_r"].numpy(), np64(inp["w13"]), np64(inp["w2"]), cfg.k,
            cfg.score, cfg.renorm, logit_bias=bias, shared=shared, z=z, given_experts=given,
            capacity=cap)
    c["z_own"] = z_own
    g = bwd(c, np64(inp["dout"]))
    if cfg.pad_to_max:  # the same kept pairs, in the static padded layout
        routed = (oracle.route(c["z"], cfg.k, cfg.score, cfg.renorm) if given is None
                  else oracle.route_replay(c["z"], given, cfg.score, cfg.renorm))
        c = dict(c, route=oracle.pad_to_max(routed, cap))
    if cfg.aux_loss_coeff > 0:
        # the auxiliary loss adds its gradient to d_logits (counts of the routing)
        L, dz = oracle.aux_loss(c["z"], c["route"]["counts"], cfg.k, cfg.score, cfg.aux_loss_coeff)
        dWr, dxr = oracle.router_logits_bwd(np64(inp["x"]), inp["w_r"].numpy(), dz)
        g = dict(g, d_logits=g["d_logits"] + dz, dW_r=g["dW_r"] + dWr, dx=g["dx"] + dxr, aux=L)
    return layer, c, g


def _check(cfg, layer, c, g):
    tol = TOL[cfg.gemm]
    r = c["route"]
    np.testing.assert_array_equal(layer.topk_idx.cpu().numpy(), r["topk_idx"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), r["offsets"])
    np.testing.assert_array_equal(layer.dst_row.cpu().numpy(), r["dst_row"])
    n_rows = int(r["offsets"][-1])
    np.testing.assert_array_equal(layer.src_token.cpu().numpy()[:n_rows], r["src_token"])
    assert_close("logits (oracle's own)", layer.logits, c["z_own"], TOL["f32"])
    assert_close("out", layer.out, c["out"], tol)
    grads = layer.grads()
    for name in ["dx", "d_logits", "dW_r", "dW13", "dW2"] + (["dWs13", "dWs2"] if cfg.fs else []):
        assert_close(name, grads[name], g[name], tol)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_tiny_fp32(gpu, seed):
    cfg = inputs.CONFIGS["tiny_fp32"]
    _check(cfg, *_run(cfg, seed))


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_BF16_SOFTMAX], ids=lambda c: c.name)
def test_layer_small_bf16(gpu, cfg):
    _check(cfg, *_run(cfg, 0))


def test_layer_tiny_fp32_with_shared_and_sigmoid(gpu):
    cfg = dataclasses.replace(inputs.CONFIGS["tiny_fp32"], name="tiny_fp32_shared", fs=64,
                              score="sigmoid", bias="normal")
    _check(cfg, *_run(cfg, 3))


def test_layer_balanced_routing_replayed(gpu):
    """Force-balanced routing (every expert exactly T*k/E rows), the experts
    given and replayed; the routing weights still come from the keys."""
    cfg = inputs.CONFIGS["small_balanced"]
    layer, c, g = _run(cfg, 0)
    assert (layer.counts.cpu().numpy() == cfg.T * cfg.k // cfg.E).all()
    assert int(layer.route_status.item()) == 0
    _check(cfg, layer, c, g)


@pytest.mark.parametrize("cfg", [SMALL_BF16, inputs.CONFIGS["small_balanced"]],
                         ids=lambda c: c.name)
def test_layer_recompute_activation(gpu, cfg):
    """H = silu(A) * B rebuilt from AB in the backward instead of kept."""
    _check(cfg, *_run(cfg, 1, recompute_act=True))


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_BF16_SOFTMAX, inputs.CONFIGS["small_balanced"]],
                         ids=lambda c: c.name)
def test_layer_gate_in_ffn(gpu, cfg):
    """Routing weight applied before W2: unweighted combine, no Y in the
    backward, the weight gradient from the GEMM 2 dgrad epilogue."""
    layer, c, g = _run(cfg, 2, gate_in_ffn=True)
    _check(cfg, layer, c, g)
    assert_close("d_topk_w", layer.d_topk_w, g["d_topk_w"], TOL[cfg.gemm])


@pytest.mark.parametrize("gated", [False, True])
def test_layer_capacity_dropping(gpu, gated):
    """Capacity-limited dropping on a skewed (Zipf-biased) routing: pairs past
    an expert's capacity are dropped and contribute nothing."""
    cfg = inputs.CONFIGS["small_capacity"]
    layer, c, g = _run(cfg, 0, gate_in_ffn=gated)
    assert (c["route"]["dst_row"] < 0).sum() > 0  # the case really drops
    _check(cfg, layer, c, g)
    assert_close("d_topk_w", layer.d_topk_w, g["d_topk_w"], TOL[cfg.gemm])


def test_layer_aux_loss(gpu):
    """Auxiliary load-balancing loss: its value, and its gradient added to the
    router's (through d_logits into dW_r and dx)."""
    cfg = inputs.CONFIGS["small_aux"]
    layer, c, g = _run(cfg, 0)
    _check(cfg, layer, c, g)
    assert abs(float(layer.aux_loss.item()) - g["aux"]) <= 1e-5 * abs(g["aux"])


def test_layer_repeat_is_bitwise_deterministic(gpu):
    cfg = SMALL_BF16
    inp = inputs.layer_inputs(cfg, 5)
    w = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    layer = MoELayer(cfg, w, DEV)
    layer.forward(w["x"])
    layer.backward(w["dout"])
    first = {k: v.clone() for k, v in layer.grads().items()}
    out1 = layer.out.clone()
    layer.forward(w["x"])
    layer.backward(w["dout"])
    assert torch.equal(out1, layer.out)
    for k, v in layer.grads().items():
        assert torch.equal(first[k], v), k


def test_layer_expert_bias(gpu):
    """Selection-only expert bias: the experts of the biased keys, the weights
    and every gradient of the layer on the unbiased scores, and the bias moved
    by the update rule (bit-exact) from the step's loads."""
    cfg = inputs.CONFIGS["small_expert_bias"]
    layer, c, g = _run(cfg, 0)
    _check(cfg, layer, c, g)
    b0 = inputs.layer_inputs(cfg, 0)["expert_bias"].numpy()
    want = oracle.expert_bias_update(b0, c["route"]["counts"], np.float32(cfg.expert_bias_rate))
    np.testing.assert_array_equal(layer.sel_bias.cpu().numpy().view(np.int32),
                                  want.view(np.int32))
    assert (want != b0).any()


@pytest.mark.parametrize("recompute", [False, True])
def test_layer_pad_to_max(gpu, recompute):
    """Every expert's segment padded to the capacity: the static padded map,
    and the layer's outputs and gradients equal to capacity dropping."""
    cfg = inputs.CONFIGS["small_pad_to_max"]
    layer, c, g = _run(cfg, 0, recompute_act=recompute)
    assert layer.x_perm.shape[0] == cfg.E * layer.capacity
    _check(cfg, layer, c, g)
