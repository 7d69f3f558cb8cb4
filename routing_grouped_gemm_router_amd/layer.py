"""One MoE layer, forward and backward, composed from the C-ABI calls.

The four stages of "Scalable Training of Mixture-of-Experts Models with
Megatron Core", section 2 (Route, Dispatch, Expert Computation, Combine), and
their backward, each one or more HIP kernels on the current stream:

  forward   moe_router_logits -> moe_route_topk -> moe_permute
            -> moe_grouped_gemm_fwd (SwiGLU epilogue) -> moe_grouped_gemm_fwd
            [-> shared expert: the same two GEMMs as one group over all tokens]
            -> moe_unpermute_combine
  backward  moe_unpermute_combine_bwd -> moe_grouped_gemm_dgrad (SwiGLU-backward
            epilogue) -> moe_grouped_gemm_wgrad -> moe_grouped_gemm_dgrad
            -> moe_grouped_gemm_wgrad [-> shared expert] -> moe_route_topk_bwd
            -> moe_router_logits_bwd -> moe_permute_bwd (+ shared and router dx)

No step synchronises with the host: per-expert row counts stay on the device
and every buffer is sized from T * k.  Buffers are allocated once per layer
and reused across steps.  Python here only allocates and orders the calls.
"""
import contextlib

import torch

from . import abi


class EventTimer:
    """Per-call device timing with HIP events on the current stream.

    ``span(name)`` brackets the enqueued calls with two events; ``summary()``
    (after a synchronize) returns name -> (mean ms per span, count)."""

    def __init__(self):
        self.spans = {}

    @contextlib.contextmanager
    def span(self, name):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.spans.setdefault(name, []).append((a, b))

    def summary(self):
        return {n: (sum(a.elapsed_time(b) for a, b in v) / len(v), len(v))
                for n, v in self.spans.items()}


_NO_SPAN = contextlib.nullcontext()


class MoELayer:
    """Holds weights, activations saved for backward, and gradients.

    weights: dict with w_r [d, E] fp32, logit_bias [E] fp32 or None,
    w13 [E, d, 2f], w2 [E, f, d] and, with a shared expert, ws13 [d, 2fs],
    ws2 [fs, d] (activation dtype)."""

    def __init__(self, cfg, weights, device="cuda"):
        self.cfg = cfg
        self.timer = None
        self.dev = torch.device(device)
        self.w = weights
        T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
        N = T * k
        dt = cfg.torch_dtype()
        dev = self.dev
        self.score = abi.SOFTMAX if cfg.score == "softmax" else abi.SIGMOID
        emp = lambda *s, dtype=dt: torch.empty(s, dtype=dtype, device=dev)  # noqa: E731
        # forward state
        self.logits = emp(T, E, dtype=torch.float32)
        self.topk_idx = emp(T, k, dtype=torch.int32)
        self.topk_w = emp(T, k, dtype=torch.float32)
        self.counts = emp(E, dtype=torch.int32)
        self.offsets = emp(E + 1, dtype=torch.int64)
        self.dst_row = emp(T, k, dtype=torch.int32)
        self.src_token = emp(N, dtype=torch.int32)
        self.route_ws = emp(abi.moe_route_topk_workspace_bytes(T, E, k), dtype=torch.uint8)
        self.x_perm = emp(N, d)
        self.ab = emp(N, 2 * f)
        self.h = emp(N, f)
        self.y = emp(N, d)
        self.out = emp(T, d)
        # backward state
        self.d_topk_w = emp(T, k, dtype=torch.float32)
        self.dy = emp(N, d)
        self.dab = emp(N, 2 * f)
        self.dx_perm = emp(N, d)
        self.dw13 = emp(E, d, 2 * f)
        self.dw2 = emp(E, f, d)
        self.d_logits = emp(T, E, dtype=torch.float32)
        self.dw_r = emp(d, E, dtype=torch.float32)
        self.dx_router = emp(T, d, dtype=torch.float32)
        self.dx = emp(T, d)
        self.shared = cfg.fs > 0
        if self.shared:
            fs = cfg.fs
            self.off_all = torch.tensor([0, T], dtype=torch.int64, device=dev)
            self.ws13 = weights["ws13"].unsqueeze(0)
            self.ws2 = weights["ws2"].unsqueeze(0)
            self.abs_ = emp(T, 2 * fs)
            self.hs = emp(T, fs)
            self.ys = emp(T, d)
            self.dabs = emp(T, 2 * fs)
            self.dxs = emp(T, d)
            self.dws13 = emp(1, d, 2 * fs)
            self.dws2 = emp(1, fs, d)

    # ------------------------------------------------------------ forward --
    def _span(self, name):
        return self.timer.span(name) if self.timer is not None else _NO_SPAN

    def forward(self, x):
        c, w = self.cfg, self.w
        self.x = x
        with self._span("router_logits"):
            abi.moe_router_logits(x, w["w_r"], w.get("logit_bias"), self.logits)
        with self._span("route_topk"):
            abi.moe_route_topk(self.logits, c.k, self.score, c.renorm, self.topk_idx, self.topk_w,
                               self.counts, self.offsets, self.dst_row, self.src_token,
                               self.route_ws)
        with self._span("permute"):
            abi.moe_permute(x, self.dst_row, self.x_perm)
        with self._span("gemm1_fwd"):
            abi.moe_grouped_gemm_fwd(self.x_perm, w["w13"], self.offsets, self.ab, self.h,
                                     epilogue=abi.EPI_SWIGLU)
        with self._span("gemm2_fwd"):
            abi.moe_grouped_gemm_fwd(self.h, w["w2"], self.offsets, self.y)
        ys = None
        if self.shared:
            with self._span("shared_gemm1_fwd"):
                abi.moe_grouped_gemm_fwd(x, self.ws13, self.off_all, self.abs_, self.hs,
                                         epilogue=abi.EPI_SWIGLU)
            with self._span("shared_gemm2_fwd"):
                abi.moe_grouped_gemm_fwd(self.hs, self.ws2, self.off_all, self.ys)
            ys = self.ys
        with self._span("combine"):
            abi.moe_unpermute_combine(self.y, self.topk_w, self.dst_row, ys, self.out)
        return self.out

    # ----------------------------------------------------------- backward --
    def backward(self, dout):
        c, w = self.cfg, self.w
        x = self.x
        with self._span("combine_bwd"):
            abi.moe_unpermute_combine_bwd(dout, self.y, self.topk_w, self.dst_row, self.dy,
                                          self.d_topk_w)
        with self._span("gemm2_dgrad"):
            abi.moe_grouped_gemm_dgrad(self.dy, w["w2"], self.offsets, self.dab,
                                       epilogue=abi.EPI_SWIGLU_BWD, ab=self.ab)
        with self._span("gemm2_wgrad"):
            abi.moe_grouped_gemm_wgrad(self.h, self.dy, self.offsets, self.dw2)
        with self._span("gemm1_dgrad"):
            abi.moe_grouped_gemm_dgrad(self.dab, w["w13"], self.offsets, self.dx_perm)
        with self._span("gemm1_wgrad"):
            abi.moe_grouped_gemm_wgrad(self.x_perm, self.dab, self.offsets, self.dw13)
        dxs = None
        if self.shared:
            with self._span("shared_gemm2_dgrad"):
                abi.moe_grouped_gemm_dgrad(dout, self.ws2, self.off_all, self.dabs,
                                           epilogue=abi.EPI_SWIGLU_BWD, ab=self.abs_)
            with self._span("shared_gemm2_wgrad"):
                abi.moe_grouped_gemm_wgrad(self.hs, dout, self.off_all, self.dws2)
            with self._span("shared_gemm1_dgrad"):
                abi.moe_grouped_gemm_dgrad(self.dabs, self.ws13, self.off_all, self.dxs)
            with self._span("shared_gemm1_wgrad"):
                abi.moe_grouped_gemm_wgrad(x, self.dabs, self.off_all, self.dws13)
            dxs = self.dxs
        with self._span("route_topk_bwd"):
            abi.moe_route_topk_bwd(self.logits, self.topk_idx, self.topk_w, self.d_topk_w,
                                   self.score, c.renorm, self.d_logits)
        with self._span("router_logits_bwd"):
            abi.moe_router_logits_bwd(x, w["w_r"], self.d_logits, self.dw_r, self.dx_router)
        with self._span("permute_bwd"):
            abi.moe_permute_bwd(self.dx_perm, self.dst_row, dxs, self.dx_router, self.dx)
        return self.dx

    def grads(self):
        g = dict(dx=self.dx, d_logits=self.d_logits, dW_r=self.dw_r, dW13=self.dw13, dW2=self.dw2,
                 d_topk_w=self.d_topk_w)
        if self.shared:
            g.update(dWs13=self.dws13[0], dWs2=self.dws2[0])
        return g
