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

With fp8 expert GEMMs (the blockwise recipe of the same report, section 5)
every expert-GEMM input is quantized on the way in: activations and gradients
in 1 x 128 tiles (moe_quant_fp8_rows), weights in 128 x 128 blocks
(moe_quant_fp8_weights, once per pass), and the operands of the weight
gradients in 128-token x 1 tiles of each expert's zero-padded rows
(moe_quant_fp8_token_tiles); routing, permute, SwiGLU and combine stay bf16 /
fp32.  With MXFP8 expert GEMMs (the same section's microscaling recipe) every
operand is blocked 1 x 32 along its contraction axis with E8M0 scales that
the matrix cores apply; the permutation is fused into the quantizers
(moe_permute_quant_mxfp8 for the forward operand, moe_quant_mxfp8_token_tiles
gathering through src_token for the weight gradient), so the permuted bf16
activations are never written.

No step synchronises with the host: per-expert row counts stay on the device
and every buffer is sized from T * k.  Buffers are allocated once per layer
and reused across steps.  Python here only allocates and orders the calls.
"""
import contextlib
import math
import os

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

    def __init__(self, cfg, weights, device="cuda", recompute_act=False, gate_in_ffn=False):
        self.cfg = cfg
        # gate_in_ffn: the routing weight scales H before W2 (moe_permute_weights,
        # moe_grouped_gemm_gated_fwd); the combine is an unweighted sum and its
        # backward a gather of dout, so Y is not needed by the backward; the
        # routing-weight gradient comes from the GEMM 2 dgrad epilogue
        # (moe_grouped_gemm_gated_dgrad, moe_gate_grad).  bf16 only.
        self.gated = gate_in_ffn
        if gate_in_ffn and (cfg.gemm != "bf16" or recompute_act):
            raise ValueError("gate_in_ffn: bf16 expert GEMMs, without recompute_act")
        # recompute_act: H = silu(A) * B is not kept from the forward to the
        # backward; the backward rebuilds it from AB (moe_swiglu).  H then lives
        # in the storage of dAB, which holds nothing until the backward.
        self.recompute = recompute_act
        self.replay = cfg.routing == "balanced"
        # selection-only expert bias (auxiliary-loss-free balancing): a copy
        # that the update after each route moves
        self.ebias = cfg.expert_bias_std > 0
        if self.ebias:
            if cfg.score != "sigmoid" or self.replay:
                raise ValueError("the expert bias applies to sigmoid top-k routing")
            self.sel_bias = weights["expert_bias"].detach().clone()
        if self.replay:
            self.topk_idx_in = weights["topk_idx_in"]
            self.route_status = torch.zeros(1, dtype=torch.int32, device=device)
        self.timer = None
        self.dev = torch.device(device)
        # MOE_CHECK_FINITE set: non-finite router logits (a caller error) raise
        # the device word finite_status to 1 (read it with finite_ok())
        self.check_finite = os.environ.get("MOE_CHECK_FINITE", "") not in ("", "0")
        if self.check_finite:
            self.finite_status = torch.zeros(1, dtype=torch.int32, device=self.dev)
        # MOE_DEBUG set: every route's dispatch map is checked against its
        # invariants before the permute and the GEMMs use it (moe_check_dispatch);
        # violations accumulate as bits in debug_status (read with dispatch_ok())
        self.debug = os.environ.get("MOE_DEBUG", "") not in ("", "0")
        if self.debug:
            self.debug_status = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.w = weights
        T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
        N = T * k
        dt = cfg.torch_dtype()
        dev = self.dev
        self.score = abi.SOFTMAX if cfg.score == "softmax" else abi.SIGMOID
        # the route's backward leaves d_logits zero off each token's chosen
        # experts with renormalised routing or sigmoid scores, unless the
        # auxiliary loss adds its dense gradient
        self.sparse_dz = ((cfg.renorm or cfg.score == "sigmoid") and cfg.aux_loss_coeff <= 0
                          and cfg.E <= 256 and cfg.d % 8 == 0)
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
        # capacity-limited dropping: the route writes the dropless map here and
        # moe_apply_capacity the kept one into counts / offsets / dst_row / src_token
        self.capacity = (int(math.ceil(cfg.capacity_factor * T * k / E))
                         if cfg.capacity_factor > 0 else None)
        self.aux = cfg.aux_loss_coeff > 0
        if self.aux:
            self.aux_loss = emp(1, dtype=torch.float32)
            self.aux_ws = emp(abi.moe_aux_loss_workspace_bytes(T, E), dtype=torch.uint8)
        # pad-to-max: every expert owns `capacity` rows at e * capacity (static
        # offsets); padding rows are kept zero in the buffers the GEMMs read
        self.pad = cfg.pad_to_max
        if self.pad and (self.capacity is None or cfg.gemm not in ("bf16", "f32") or gate_in_ffn):
            raise ValueError("pad_to_max: needs a capacity, bf16 / fp32 GEMMs, no gate_in_ffn")
        if self.pad:
            N = E * self.capacity  # rows of the permuted buffers
            self.src_token = emp(N, dtype=torch.int32)
        if self.capacity is not None:
            self.full = dict(counts=emp(E, dtype=torch.int32), offsets=emp(E + 1, dtype=torch.int64),
                             dst_row=emp(T, k, dtype=torch.int32),
                             src_token=emp(T * k, dtype=torch.int32))
        # the MXFP8 path gathers x inside its quantizers: no permuted bf16 copy
        self.x_perm = emp(N, d) if cfg.gemm != "mxfp8" else None
        self.ab = emp(N, 2 * f)
        self.y = emp(N, d)
        self.out = emp(T, d)
        # backward state
        self.d_topk_w = emp(T, k, dtype=torch.float32)
        self.dy = emp(N, d)
        self.dab = emp(N, 2 * f)
        self.h = self.dab.view(-1)[:N * f].view(N, f) if recompute_act else emp(N, f)
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
        if self.gated:
            self.w_perm = emp(N, dtype=torch.float32)
            self.gate_part = emp(N, f // 64, dtype=torch.float32)
        self.lowp = cfg.gemm if cfg.gemm in ("fp8", "mxfp8") else None
        self.mx = cfg.gemm == "mxfp8"
        if self.lowp:
            self._alloc_lowp()

    def _alloc_lowp(self):
        c, dev, mx = self.cfg, self.dev, self.mx
        T, d, E, k, f, fs = c.T, c.d, c.E, c.k, c.f, c.fs
        N = T * k
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
        if mx:
            self._gemm = dict(fwd=abi.moe_grouped_gemm_mxfp8_fwd,
                              dgrad=abi.moe_grouped_gemm_mxfp8_dgrad,
                              wgrad=abi.moe_grouped_gemm_mxfp8_wgrad)
        else:
            self._gemm = dict(fwd=abi.moe_grouped_gemm_fp8_fwd,
                              dgrad=abi.moe_grouped_gemm_fp8_dgrad,
                              wgrad=abi.moe_grouped_gemm_fp8_wgrad)

        def wq(G, K, Nn):  # the operands of a [G, K, N] weight in each GEMM
            if mx:  # E8M0 bytes per 32 along each layout's contraction axis
                return dict(qf=u8(G, Nn, K), sf=u8(G, Nn, K // 32), qd=u8(G, K, Nn),
                            sd=u8(G, K, Nn // 32))
            # blockwise: one code array in the weight's own layout serves both
            q = u8(G, K, Nn)
            return dict(qf=q, sf=f32(G, K // 128, Nn), qd=q, sd=f32(G, Nn // 128, K))

        def rows(M, K):  # 1 x 128 row tiles (MX: 1 x 32 blocks)
            if mx:
                return dict(q=u8(M, K), s=u8(M, K // 32))
            return dict(q=u8(M, K), s=f32(K // 128, M))

        self.q = dict(w13=wq(E, d, 2 * f), w2=wq(E, f, d), x=rows(N, d), h=rows(N, f),
                      dy=rows(N, d), dab=rows(N, 2 * f))
        self.ldm = abi.moe_padded_rows_bound(N, E, 128)
        self.poff = torch.empty(E + 1, dtype=torch.int64, device=dev)

        def tiles(K, ldm):  # 128-token x 1 tiles (MX: 32-token blocks), transposed
            if mx:
                return dict(q=u8(K, ldm), s=u8(K, ldm // 32))
            return dict(q=u8(K, ldm), s=f32(ldm // 128, K))

        self.qt = dict(x=tiles(d, self.ldm), dab=tiles(2 * f, self.ldm), h=tiles(f, self.ldm),
                       dy=tiles(d, self.ldm))
        if self.shared:
            self.ldm_s = abi.moe_padded_rows_bound(T, 1, 128)
            self.poff_all = torch.tensor([0, (T + 127) // 128 * 128], dtype=torch.int64,
                                         device=dev)
            self.q.update(ws13=wq(1, d, 2 * fs), ws2=wq(1, fs, d), xs=rows(T, d), hs=rows(T, fs),
                          douts=rows(T, d), dabs=rows(T, 2 * fs))
            self.qt.update(xs=tiles(d, self.ldm_s), dabs=tiles(2 * fs, self.ldm_s),
                           hs=tiles(fs, self.ldm_s), douts=tiles(d, self.ldm_s))

    # ------------------------------------------------- fp8 and MXFP8 ---
    def _qrows(self, name, a):
        if self.mx:
            abi.moe_quant_mxfp8_rows(a, self.q[name]["q"], self.q[name]["s"])
        else:
            abi.moe_quant_fp8_rows(a, self.q[name]["q"], self.q[name]["s"])
        return self.q[name]["q"], self.q[name]["s"]

    def _qtiles(self, name, a, offsets, poff, src_row=None):
        t = self.qt[name]
        if self.mx:
            abi.moe_quant_mxfp8_token_tiles(a, offsets, poff, t["q"], t["s"], src_row=src_row,
                                            M=self.cfg.N)
        else:
            abi.moe_quant_fp8_token_tiles(a, offsets, poff, t["q"], t["s"])
        return t["q"], t["s"]

    def _qweights(self, name, w):
        t = self.q[name]
        if self.mx:
            abi.moe_quant_mxfp8_weights(w, t["qf"], t["sf"], t["qd"], t["sd"])
        else:
            abi.moe_quant_fp8_weights(w, t["qd"], t["sf"], t["sd"])

    def _forward_lowp(self, x):
        c, w, q, gm = self.cfg, self.w, self.q, self._gemm
        with self._span("quant_weights"):
            self._qweights("w13", w["w13"])
            self._qweights("w2", w["w2"])
            if self.shared:
                self._qweights("ws13", self.ws13)
                self._qweights("ws2", self.ws2)
        if self.mx:
            with self._span("permute_quant_x"):
                # every row below offsets[E] has exactly one slot (no padding
                # rows: pad-to-max is bf16 / fp32 only), so the token-side
                # scatter gives the gather's bytes with one read of x
                abi.moe_scatter_quant_mxfp8(x, self.dst_row, self.offsets, q["x"]["q"],
                                            q["x"]["s"])
                xq, xs = q["x"]["q"], q["x"]["s"]
        else:
            with self._span("quant_x"):
                xq, xs = self._qrows("x", self.x_perm)
        with self._span("gemm1_fwd"):
            gm["fwd"](xq, xs, q["w13"]["qf"], q["w13"]["sf"], self.offsets, self.ab, self.h,
                      epilogue=abi.EPI_SWIGLU)
        with self._span("quant_h"):
            hq, hs = self._qrows("h", self.h)
        with self._span("gemm2_fwd"):
            gm["fwd"](hq, hs, q["w2"]["qf"], q["w2"]["sf"], self.offsets, self.y)
        if self.shared:
            with self._span("shared_quant_x"):
                xq_, xs_ = self._qrows("xs", x)
            with self._span("shared_gemm1_fwd"):
                gm["fwd"](xq_, xs_, q["ws13"]["qf"], q["ws13"]["sf"], self.off_all, self.abs_,
                          self.hs, epilogue=abi.EPI_SWIGLU)
            with self._span("shared_quant_h"):
                hq_, hs_ = self._qrows("hs", self.hs)
            with self._span("shared_gemm2_fwd"):
                gm["fwd"](hq_, hs_, q["ws2"]["qf"], q["ws2"]["sf"], self.off_all, self.ys)

    def _backward_lowp(self, dout):
        q, x, gm = self.q, self.x, self._gemm

        def gemm2_dgrad():
            with self._span("quant_dy"):
                dyq, dys = self._qrows("dy", self.dy)
            with self._span("gemm2_dgrad"):
                gm["dgrad"](dyq, dys, q["w2"]["qd"], q["w2"]["sd"], self.offsets, self.dab,
                            epilogue=abi.EPI_SWIGLU_BWD, ab=self.ab)

        def gemm2_wgrad():
            with self._span("quant_tiles_h_dy"):
                abi.moe_padded_offsets(self.offsets, self.cfg.N, self.poff)
                hT, hTs = self._qtiles("h", self.h, self.offsets, self.poff)
                dyT, dyTs = self._qtiles("dy", self.dy, self.offsets, self.poff)
            with self._span("gemm2_wgrad"):
                gm["wgrad"](hT, hTs, dyT, dyTs, self.poff, self.dw2)

        if self.recompute:  # H in dAB's storage: use it before the dgrad writes dAB
            with self._span("swiglu_recompute"):
                abi.moe_swiglu(self.ab, self.h)
            gemm2_wgrad()
            gemm2_dgrad()
        else:
            gemm2_dgrad()
            gemm2_wgrad()
        with self._span("quant_dab"):
            dabq, dabs = self._qrows("dab", self.dab)
        with self._span("gemm1_dgrad"):
            gm["dgrad"](dabq, dabs, q["w13"]["qd"], q["w13"]["sd"], self.offsets, self.dx_perm)
        with self._span("quant_tiles_x_dab"):
            if self.mx:  # x's rows gathered through the permutation
                xT, xTs = self._qtiles("x", x, self.offsets, self.poff, src_row=self.src_token)
            else:
                xT, xTs = self._qtiles("x", self.x_perm, self.offsets, self.poff)
            dabT, dabTs = self._qtiles("dab", self.dab, self.offsets, self.poff)
        with self._span("gemm1_wgrad"):
            gm["wgrad"](xT, xTs, dabT, dabTs, self.poff, self.dw13)
        if self.shared:
            with self._span("shared_quant_dout"):
                dq, ds = self._qrows("douts", dout)
            with self._span("shared_gemm2_dgrad"):
                gm["dgrad"](dq, ds, q["ws2"]["qd"], q["ws2"]["sd"], self.off_all, self.dabs,
                            epilogue=abi.EPI_SWIGLU_BWD, ab=self.abs_)
            with self._span("shared_quant_tiles_h_dout"):
                a, sa = self._qtiles("hs", self.hs, self.off_all, self.poff_all)
                b, sb = self._qtiles("douts", dout, self.off_all, self.poff_all)
            with self._span("shared_gemm2_wgrad"):
                gm["wgrad"](a, sa, b, sb, self.poff_all, self.dws2)
            with self._span("shared_quant_dab"):
                dq, ds = self._qrows("dabs", self.dabs)
            with self._span("shared_gemm1_dgrad"):
                gm["dgrad"](dq, ds, q["ws13"]["qd"], q["ws13"]["sd"], self.off_all, self.dxs)
            with self._span("shared_quant_tiles_x_dab"):
                a, sa = self._qtiles("xs", x, self.off_all, self.poff_all)
                b, sb = self._qtiles("dabs", self.dabs, self.off_all, self.poff_all)
            with self._span("shared_gemm1_wgrad"):
                gm["wgrad"](a, sa, b, sb, self.poff_all, self.dws13)

    def dispatch_ok(self):
        """The bits moe_check_dispatch raised in every forward so far (0: none);
        MOE_DEBUG must have been set when the layer was built.  Synchronises."""
        if not self.debug:
            raise RuntimeError("MOE_DEBUG was not set when the layer was built")
        return int(self.debug_status.item())

    def finite_ok(self):
        """False once a forward met a non-finite logit (MOE_CHECK_FINITE set);
        reads the device status word, so it synchronises."""
        if not self.check_finite:
            raise RuntimeError("MOE_CHECK_FINITE was not set when the layer was built")
        return int(self.finite_status.item()) == 0

    # ------------------------------------------------------------ forward --
    def _span(self, name):
        return self.timer.span(name) if self.timer is not None else _NO_SPAN

    def forward(self, x):
        c, w = self.cfg, self.w
        self.x = x
        with self._span("router_logits"):
            abi.moe_router_logits(x, w["w_r"], w.get("logit_bias"), self.logits)
        if self.check_finite:
            abi.moe_check_finite(self.logits, self.finite_status)
        with self._span("route_topk"):
            m = self.full if self.capacity is not None else dict(
                counts=self.counts, offsets=self.offsets, dst_row=self.dst_row,
                src_token=self.src_token)
            if self.replay:
                abi.moe_route_replay(self.logits, self.topk_idx_in, self.score, c.renorm,
                                     self.topk_idx, self.topk_w, m["counts"], m["offsets"],
                                     m["dst_row"], m["src_token"], self.route_ws,
                                     status=self.route_status)
            elif self.ebias:
                abi.moe_route_topk_expert_bias(self.logits, self.sel_bias, c.k, c.renorm,
                                               self.topk_idx, self.topk_w, m["counts"],
                                               m["offsets"], m["dst_row"], m["src_token"],
                                               self.route_ws)
            else:
                abi.moe_route_topk(self.logits, c.k, self.score, c.renorm, self.topk_idx,
                                   self.topk_w, m["counts"], m["offsets"], m["dst_row"],
                                   m["src_token"], self.route_ws)
            if self.pad:
                abi.moe_pad_to_max(self.topk_idx, m["counts"], m["offsets"], m["dst_row"],
                                   m["src_token"], self.capacity, self.counts, self.offsets,
                                   self.dst_row, self.src_token)
            elif self.capacity is not None:
                abi.moe_apply_capacity(self.topk_idx, m["counts"], m["offsets"], m["dst_row"],
                                       self.capacity, self.counts, self.offsets, self.dst_row,
                                       self.src_token)
        if self.debug:
            abi.moe_check_dispatch(self.topk_idx, self.counts, self.offsets, self.dst_row,
                                   self.src_token, self.src_token.numel(), self.debug_status)
        self.routed_counts = m["counts"]  # before any dropping
        self.route_map = m                # the dropless dispatch map
        if self.ebias and c.expert_bias_rate > 0:  # the next route sees the moved bias
            with self._span("expert_bias_update"):
                abi.moe_expert_bias_update(self.routed_counts, c.expert_bias_rate, self.sel_bias)
        if self.aux:
            with self._span("aux_loss"):
                abi.moe_aux_loss(self.logits, self.routed_counts, c.k, self.score,
                                 c.aux_loss_coeff, loss=self.aux_loss, workspace=self.aux_ws)
        if not self.mx:
            with self._span("permute"):
                abi.moe_permute(x, self.dst_row, self.x_perm)
                if self.pad:
                    abi.moe_zero_unmapped_rows(self.x_perm, self.src_token)
        if self.lowp:
            self._forward_lowp(x)
            with self._span("combine"):
                abi.moe_unpermute_combine(self.y, self.topk_w, self.dst_row,
                                          self.ys if self.shared else None, self.out)
            return self.out
        if self.gated:
            with self._span("permute_weights"):
                abi.moe_permute_weights(self.topk_w, self.dst_row, self.w_perm)
            with self._span("gemm1_fwd"):
                abi.moe_grouped_gemm_gated_fwd(self.x_perm, w["w13"], self.offsets, self.w_perm,
                                               self.ab, self.h)
        else:
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
            abi.moe_unpermute_combine(self.y, None if self.gated else self.topk_w, self.dst_row,
                                      ys, self.out)
        return self.out

    # ----------------------------------------------------------- backward --
    def backward(self, dout):
        c, w = self.cfg, self.w
        x = self.x
        with self._span("combine_bwd"):
            if self.gated:  # unweighted combine: its backward gathers dout
                abi.moe_permute(dout, self.dst_row, self.dy)
            else:
                abi.moe_unpermute_combine_bwd(dout, self.y, self.topk_w, self.dst_row, self.dy,
                                              self.d_topk_w)
                if self.pad:
                    abi.moe_zero_unmapped_rows(self.dy, self.src_token)
        if self.lowp:
            self._backward_lowp(dout)
            return self._backward_tail(dout, self.dxs if self.shared else None)
        if self.gated:
            with self._span("gemm2_dgrad"):
                abi.moe_grouped_gemm_gated_dgrad(self.dy, w["w2"], self.offsets, self.ab,
                                                 self.w_perm, self.dab, self.gate_part)
            with self._span("gate_grad"):
                abi.moe_gate_grad(self.gate_part, self.dst_row, self.d_topk_w)
            with self._span("gemm2_wgrad"):
                abi.moe_grouped_gemm_wgrad(self.h, self.dy, self.offsets, self.dw2)
        elif self.recompute:
            # H again from AB, into dAB's storage; used by the weight gradient
            # before the dgrad overwrites that storage with dAB
            with self._span("swiglu_recompute"):
                abi.moe_swiglu(self.ab, self.h)
            with self._span("gemm2_wgrad"):
                abi.moe_grouped_gemm_wgrad(self.h, self.dy, self.offsets, self.dw2)
            with self._span("gemm2_dgrad"):
                abi.moe_grouped_gemm_dgrad(self.dy, w["w2"], self.offsets, self.dab,
                                           epilogue=abi.EPI_SWIGLU_BWD, ab=self.ab)
        else:
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
        return self._backward_tail(dout, dxs)

    def _backward_tail(self, dout, dxs):
        c, w, x = self.cfg, self.w, self.x
        with self._span("route_topk_bwd"):
            abi.moe_route_topk_bwd(self.logits, self.topk_idx, self.topk_w, self.d_topk_w,
                                   self.score, c.renorm, self.d_logits)
        if self.aux:  # the loss's gradient is added to d_logits
            with self._span("aux_loss_bwd"):
                abi.moe_aux_loss(self.logits, self.routed_counts, c.k, self.score,
                                 c.aux_loss_coeff, d_logits=self.d_logits)
        with self._span("router_logits_bwd"):
            if self.sparse_dz:
                # d_logits is zero off each token's chosen experts: only those entries are read
                abi.moe_router_logits_bwd_topk(x, w["w_r"], self.d_logits, self.topk_idx,
                                               self.route_map["offsets"],
                                               self.route_map["src_token"], self.dw_r,
                                               self.dx_router)
            else:
                abi.moe_router_logits_bwd(x, w["w_r"], self.d_logits, self.dw_r, self.dx_router)
        with self._span("permute_bwd"):
            abi.moe_permute_bwd(self.dx_perm, self.dst_row, dxs, self.dx_router, self.dx)
        return self.dx

    def data_movement_calls(self, dout):
        """The layer's permute / combine calls and their backward, as issued in
        the last step (same buffers, same arguments), one closure each, for
        timing them on their own.  Valid after a forward and a backward."""
        calls = {}
        if self.x_perm is not None and not self.pad:
            calls["permute"] = lambda: abi.moe_permute(self.x, self.dst_row, self.x_perm)
        ys = self.ys if self.shared else None
        calls["combine"] = lambda: abi.moe_unpermute_combine(
            self.y, None if self.gated else self.topk_w, self.dst_row, ys, self.out)
        if self.gated:
            calls["combine_bwd"] = lambda: abi.moe_permute(dout, self.dst_row, self.dy)
        else:
            calls["combine_bwd"] = lambda: abi.moe_unpermute_combine_bwd(
                dout, self.y, self.topk_w, self.dst_row, self.dy, self.d_topk_w)
        dxs = self.dxs if self.shared else None
        calls["permute_bwd"] = lambda: abi.moe_permute_bwd(self.dx_perm, self.dst_row, dxs,
                                                           self.dx_router, self.dx)
        return calls

    def grads(self):
        g = dict(dx=self.dx, d_logits=self.d_logits, dW_r=self.dw_r, dW13=self.dw13, dW2=self.dw2,
                 d_topk_w=self.d_topk_w)
        if self.shared:
            g.update(dWs13=self.dws13[0], dWs2=self.dws2[0])
        return g
