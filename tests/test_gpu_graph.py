"""The layer step is host-sync-free and allocation-free after construction,
so a whole forward + backward can be captured in a HIP graph (the role CUDA
Graphs play in "Scalable Training of Mixture-of-Experts Models with Megatron
Core", section 7, for the launch-bound MoE pieces).  Each replay, with fresh
inputs copied into the captured buffers and eager work in between, must equal
the eager step on the same inputs bit for bit (the kernels are
deterministic)."""
import dataclasses

import pytest
import torch

from routing_grouped_gemm_router_amd import inputs
from routing_grouped_gemm_router_amd.layer import MoELayer

pytestmark = pytest.mark.gpu
DEV = "cuda"

BASE = inputs.LayerConfig("graph_bf16", T=384, d=256, E=8, k=2, f=256, fs=128, score="sigmoid",
                          bias="normal")
CASES = [BASE,
         dataclasses.replace(BASE, name="graph_capacity_pad", score="softmax", bias="zipf",
                             capacity_factor=1.0, pad_to_max=True),
         dataclasses.replace(BASE, name="graph_mxfp8", gemm="mxfp8", T=512),
         dataclasses.replace(BASE, name="graph_fp8", gemm="fp8")]


def _outputs(layer):
    g = layer.grads()
    outs = {"out": layer.out, "logits": layer.logits, "topk_idx": layer.topk_idx, **g}
    return {k: v.detach().clone() for k, v in outs.items()}


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_layer_step_replays_in_a_graph(gpu, cfg):
    print(f"graph capture {cfg.name}", flush=True)
    inp = inputs.layer_inputs(cfg, 0, DEV)
    layer = MoELayer(cfg, inp, DEV)
    x = inp["x"].clone()
    dout = inp["dout"].clone()
    feeds = [(inputs.layer_inputs(cfg, s, DEV)["x"], inputs.layer_inputs(cfg, s, DEV)["dout"])
             for s in (1, 2, 3)]

    # eager reference for every feed
    want = []
    for fx, fd in feeds:
        x.copy_(fx)
        dout.copy_(fd)
        layer.forward(x)
        layer.backward(dout)
        torch.cuda.synchronize()
        want.append(_outputs(layer))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side
        layer.forward(x)
        layer.backward(dout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x)
        layer.backward(dout)
    torch.cuda.synchronize()

    for i, (fx, fd) in enumerate(feeds):
        x.copy_(fx)
        dout.copy_(fd)
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(layer)
        for name, ref in want[i].items():
            assert torch.equal(got[name], ref), f"replay {i}: {name} differs from the eager step"
        # eager work between replays on the same buffers
        layer.forward(x)
        torch.cuda.synchronize()
