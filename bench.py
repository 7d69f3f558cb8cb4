#!/usr/bin/env python3
"""Benchmark of one MoE layer, forward + backward, on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--seed S] [--no-cpu-baseline]

Default workload: the DeepSeek-V3-shaped layer (T=8192 tokens, d=7168, 256
routed SwiGLU experts with ffn 2048, sigmoid top-8 renormalised over k, one
shared expert of ffn 2048; bf16 storage, fp32 accumulation; fp32 router).
Inputs are seeded synthetic tensors generated on the GPU; weights resident in
HBM before the timed region.  A step is the whole hot path: router, top-k,
permute, both grouped GEMMs (SwiGLU fused), shared expert, combine, and the
backward of every one of them.

Also times the fp8 variants: E4M3 with fp32 block scales (``--config
deepseek_v3_fp8``) and MXFP8 (``--config deepseek_v3_mxfp8``).

Prints ONE JSON line.  ``value`` is the layer's algorithmic FLOP rate (expert
GEMM FLOPs over the routed rows plus the fp32 router FLOPs, divided by the
measured time per step).  Per-call times come from HIP events recorded on the
launch stream inside the timed region; ``roofline`` reports the dominant
kernel against MI355X's published peaks; ``cpu_baseline`` times the CPU
oracle on a bounded token sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd+bwd TFLOPS + permute/combine GB/s on 1 MI355X (roofline %)"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0     # dense fp8 MFMA, published
PEAK_F32_TFLOPS = 157.3      # fp32 vector, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="deepseek_v3_e256k8")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recompute-act", action="store_true",
                    help="rebuild H = silu(A) * B in the backward instead of keeping it")
    ap.add_argument("--gate-in-ffn", action="store_true",
                    help="apply the routing weight before W2 (unweighted combine, no Y in the "
                         "backward)")
    ap.add_argument("--cold-reps", type=int, default=5,
                    help="repetitions of each permute / combine call timed after a flush that "
                         "evicts its operands from the caches (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES once device to device (the reference that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--vendor-grouped-mm", action="store_true",
                    help="only time torch._grouped_mm (the vendor grouped GEMM) beside this "
                         "library's bf16 grouped GEMMs (plain epilogue) on the layer's own "
                         "routing of --config, print one JSON line and exit")
    return ap.parse_args()


def vendor_grouped_mm(cfg, seed, reps=5):
    """GEMM 1's three products (forward, data and weight gradient) on the
    routed rows of one forward, by this library and by torch._grouped_mm,
    HIP-event timed (median of `reps` after 2 warm-ups), with the largest
    difference between the two results relative to the largest magnitude."""
    import torch
    from routing_grouped_gemm_router_amd import abi, inputs
    from routing_grouped_gemm_router_amd.layer import MoELayer

    def timed(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    inp = inputs.layer_inputs(cfg, seed, "cuda")
    layer = MoELayer(cfg, inp, "cuda")
    layer.forward(inp["x"])
    torch.cuda.synchronize()
    off, A, W = layer.offsets, layer.x_perm, layer.w["w13"]  # A [N, d], W [E, d, 2f]
    N, d, E, f2 = A.shape[0], cfg.d, cfg.E, 2 * cfg.f
    ends = off[1:].to(torch.int32).contiguous()
    flops = 2.0 * N * d * f2
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    dC = torch.randn(N, f2, device="cuda", generator=g).to(torch.bfloat16)
    C = torch.empty(N, f2, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(N, d, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(E, d, f2, dtype=torch.bfloat16, device="cuda")
    WT = W.transpose(1, 2).contiguous()  # both libraries get contiguous operands
    AT = A.t().contiguous()
    cases = {
        "fwd": (lambda: abi.moe_grouped_gemm_fwd(A, W, off, C), C,
                lambda: torch._grouped_mm(A, W, offs=ends)),
        "dgrad": (lambda: abi.moe_grouped_gemm_dgrad(dC, W, off, dA), dA,
                  lambda: torch._grouped_mm(dC, WT, offs=ends)),
        "wgrad": (lambda: abi.moe_grouped_gemm_wgrad(A, dC, off, dW), dW,
                  lambda: torch._grouped_mm(AT, dC, offs=ends)),
    }
    rec = {"workload": cfg.name, "rows": N, "d": d, "E": E, "2f": f2}
    for name, (ours, out, vendor) in cases.items():
        t = timed(ours)
        rec[f"{name}_ms"] = round(t, 3)
        rec[f"{name}_TFLOP/s"] = round(flops / t / 1e9, 1)
        ref = vendor()
        torch.cuda.synchronize()
        rec[f"{name}_rel_diff"] = float((out.float() - ref.float()).abs().max()
                                        / ref.float().abs().max())
        t = timed(vendor)
        rec[f"vendor_{name}_ms"] = round(t, 3)
        rec[f"vendor_{name}_TFLOP/s"] = round(flops / t / 1e9, 1)
    return rec


def kernel_work(cfg, n_nonempty, gated=False, n_rows=None, sparse_router_bwd=False):
    """Algorithmic FLOPs and HBM bytes per call of every span.

    FLOPs: 2 per multiply-add over the routed rows only: the (token, slot)
    pairs that have a row, n_rows (T * k when dropless; the kept pairs under
    a capacity, whose padding rows are not counted).  Bytes: every operand
    read once and every result written once; an expert's weights count once
    per GEMM pass when the expert received rows; index and routing-weight
    arrays included.  With sparse_router_bwd (d_logits zero outside each
    token's k chosen experts, as the layer's renormalised or sigmoid routing
    without the auxiliary loss gives) the router's backward products count
    the T * k chosen entries only: the others are exact zeros."""
    T, d, E, k, f, fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs
    N = T * k if n_rows is None else n_rows
    s = 2 if cfg.dtype == "bf16" else 4      # activation / weight element bytes
    w13 = n_nonempty * d * 2 * f * s
    w2 = n_nonempty * f * d * s
    idx = T * k * 4
    w = {
        "router_logits": (2.0 * T * d * E, T * d * s + d * E * 4 + T * E * 4),
        "route_topk": (0.0, T * E * 4 + 3 * idx + T * k * 4 + N * 4),
        "permute": (0.0, T * d * s + idx + N * d * s),
        "gemm1_fwd": (2.0 * N * d * 2 * f, N * d * s + w13 + N * 2 * f * s + N * f * s),
        "gemm2_fwd": (2.0 * N * f * d, N * f * s + w2 + N * d * s),
        "combine": (0.0, N * d * s + 2 * idx + T * d * s * (2 if fs else 1)),
        "combine_bwd": (0.0, T * d * s + 2 * N * d * s + 3 * idx),
        "gemm2_dgrad": (2.0 * N * d * f, N * d * s + w2 + N * 2 * f * s * 2),
        "gemm2_wgrad": (2.0 * N * f * d, N * f * s + N * d * s + E * f * d * s),
        "gemm1_dgrad": (2.0 * N * 2 * f * d, N * 2 * f * s + w13 + N * d * s),
        "gemm1_wgrad": (2.0 * N * d * 2 * f, N * d * s + N * 2 * f * s + E * d * 2 * f * s),
        "route_topk_bwd": (0.0, T * E * 4 * 2 + 3 * idx),
        "expert_bias_update": (0.0, E * 4 * 3),
        "swiglu_recompute": (0.0, N * 2 * f * s + N * f * s),
        "router_logits_bwd": ((4.0 * T * k * d, T * d * s + 3 * idx + N * 4 + d * E * 4 * 2 + T * d * 4)
                              if sparse_router_bwd else
                              (4.0 * T * d * E, T * d * s + T * E * 4 + d * E * 4 * 2 + T * d * 4)),
        "permute_bwd": (0.0, N * d * s + idx + T * d * (s + 4 + (s if fs else 0))),
    }
    if cfg.gemm in ("fp8", "mxfp8"):
        w.update(fp8_work(cfg, n_nonempty, mx=cfg.gemm == "mxfp8", n_rows=N))
        return w
    if gated:
        # routing weight inside the expert: the combine backward is a gather of
        # dout (no Y, no dot products); GEMM 2 dgrad also writes the gate partials
        w.update({
            "permute_weights": (0.0, 2 * idx + N * 4),
            "combine_bwd": (0.0, T * d * s + idx + N * d * s),
            "gate_grad": (0.0, N * (f // 64) * 4 + idx + N * 4),
        })
        fl, by = w["gemm2_dgrad"]
        w["gemm2_dgrad"] = (fl, by + N * 4 + N * (f // 64) * 4)
    if fs:
        w.update({
            "shared_gemm1_fwd": (2.0 * T * d * 2 * fs, T * d * s + d * 2 * fs * s + T * 3 * fs * s),
            "shared_gemm2_fwd": (2.0 * T * fs * d, T * fs * s + fs * d * s + T * d * s),
            "shared_gemm2_dgrad": (2.0 * T * d * fs, T * d * s + fs * d * s + T * 4 * fs * s),
            "shared_gemm2_wgrad": (2.0 * T * fs * d, T * fs * s + T * d * s + fs * d * s),
            "shared_gemm1_dgrad": (2.0 * T * 2 * fs * d, T * 2 * fs * s + d * 2 * fs * s + T * d * s),
            "shared_gemm1_wgrad": (2.0 * T * d * 2 * fs, T * d * s + T * 2 * fs * s + d * 2 * fs * s),
        })
    return w


def fp8_work(cfg, n_nonempty, mx=False, n_rows=None):
    """FLOPs and bytes of the spans of the fp8 expert paths.  Activations are
    stored in bf16 (2 bytes) and quantized to 1-byte E4M3 codes before each
    GEMM, with one fp32 scale per 128 elements (blockwise) or one E8M0 byte per
    32 (MXFP8); weights are re-quantized every step (they change every step),
    blockwise to one code array in the weight's own layout (the forward reads
    it transposed) with the block scale expanded for each GEMM, MXFP8 to two
    copies (E8M0 scales along each GEMM's reduction); GEMM outputs are bf16.
    MXFP8 fuses the permutation into its quantizers of x (x read once, the
    row map read, no permuted bf16 copy)."""
    T, d, E, k, f, fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs
    N = T * k if n_rows is None else n_rows

    def q(n):            # bytes of n fp8 codes with their scales
        return n + (n / 32 if mx else n / 128 * 4)

    def rows(m, n):      # bf16 in, fp8 rows out
        return m * n * 2 + q(m * n)

    def wq(n):           # bf16 weight in; codes once (MXFP8: twice) and both scale vectors out
        return n * 2 + (2 * q(n) if mx else n + 2 * (n / 128 * 4))

    w13, w2 = n_nonempty * d * 2 * f, n_nonempty * f * d
    w = {
        "quant_weights": (0.0, wq(E * d * 2 * f) + wq(E * f * d)
                          + (wq(d * 2 * fs) + wq(fs * d) if fs else 0)),
        "quant_x": (0.0, rows(N, d)),
        "gemm1_fwd": (2.0 * N * d * 2 * f, q(N * d) + q(w13) + N * 2 * f * 2 + N * f * 2),
        "quant_h": (0.0, rows(N, f)),
        "gemm2_fwd": (2.0 * N * f * d, q(N * f) + q(w2) + N * d * 2),
        "quant_dy": (0.0, rows(N, d)),
        "gemm2_dgrad": (2.0 * N * d * f, q(N * d) + q(w2) + N * 2 * f * 2 * 2),
        "quant_tiles_h_dy": (0.0, rows(N, f) + rows(N, d)),
        "gemm2_wgrad": (2.0 * N * f * d, q(N * f) + q(N * d) + E * f * d * 2),
        "quant_dab": (0.0, rows(N, 2 * f)),
        "gemm1_dgrad": (2.0 * N * 2 * f * d, q(N * 2 * f) + q(w13) + N * d * 2),
        "quant_tiles_x_dab": (0.0, rows(N, d) + rows(N, 2 * f)),
        "gemm1_wgrad": (2.0 * N * d * 2 * f, q(N * d) + q(N * 2 * f) + E * d * 2 * f * 2),
    }
    if fs:
        w.update({
            "shared_quant_x": (0.0, rows(T, d)),
            "shared_gemm1_fwd": (2.0 * T * d * 2 * fs, q(T * d) + q(d * 2 * fs) + T * 3 * fs * 2),
            "shared_quant_h": (0.0, rows(T, fs)),
            "shared_gemm2_fwd": (2.0 * T * fs * d, q(T * fs) + q(fs * d) + T * d * 2),
            "shared_quant_dout": (0.0, rows(T, d)),
            "shared_gemm2_dgrad": (2.0 * T * d * fs, q(T * d) + q(fs * d) + T * 4 * fs * 2),
            "shared_quant_tiles_h_dout": (0.0, rows(T, fs) + rows(T, d)),
            "shared_gemm2_wgrad": (2.0 * T * fs * d, q(T * fs) + q(T * d) + fs * d * 2),
            "shared_quant_dab": (0.0, rows(T, 2 * fs)),
            "shared_gemm1_dgrad": (2.0 * T * 2 * fs * d, q(T * 2 * fs) + q(d * 2 * fs) + T * d * 2),
            "shared_quant_tiles_x_dab": (0.0, rows(T, d) + rows(T, 2 * fs)),
            "shared_gemm1_wgrad": (2.0 * T * d * 2 * fs, q(T * d) + q(T * 2 * fs) + d * 2 * fs * 2),
        })
    if mx:
        gather = T * d * 2 + N * 4 + q(N * d)
        w["permute_quant_x"] = (0.0, gather)
        w["quant_tiles_x_dab"] = (0.0, gather + rows(N, 2 * f))
    return w


def traffic_for(workload, kernel):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy of known size) for this workload and kernel,
    if the committed measurement was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload}/{kernel}")
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, "routing_grouped_gemm_router_amd", "csrc", src), "rb").read())
    if h.hexdigest() != rec["sha256"]:
        return None
    return rec["bytes_per_launch"]


def cold_data_movement(layer, dout, work, reps, clean=True):
    """Each permute / combine call of the layer timed on its own after a
    flush that evicts its operands from the caches, so that its reads come
    from HBM; the flush sits outside the call's events.  The flush writes
    512 MiB (twice the memory-side cache); with ``clean`` it then reads
    another 512 MiB, so the caches hold no dirty lines whose write-back the
    timed call would pay for.  Returns name -> {ms (median), GB/s, frac of
    the HBM peak}, plus their total."""
    import statistics

    import torch
    fa = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    fb = torch.ones(512 << 20, dtype=torch.uint8, device="cuda") if clean else None
    calls = layer.data_movement_calls(dout)
    res = {}
    for name, call in calls.items():
        times = []
        for _ in range(reps):
            fa.fill_(1)
            if clean:
                fb.sum(dtype=torch.int64)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = statistics.median(times)
        by = work[name][1]
        res[name] = {"ms": round(ms, 4), "GB/s": round(by / ms / 1e6, 1),
                     "frac_hbm_peak": round(by / ms / 1e6 / PEAK_HBM_GBS, 4)}
    c_ms = sum(v["ms"] for v in res.values())
    c_by = sum(work[n][1] for n in res)
    res["total"] = {"ms": round(c_ms, 4), "GB/s": round(c_by / c_ms / 1e6, 1),
                    "frac_hbm_peak": round(c_by / c_ms / 1e6 / PEAK_HBM_GBS, 4)}
    del fa, fb
    return res


def cpu_identity():
    """Cores this process may run on, and the host CPU's model name."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(cfg, inp, budget_s):
    """The CPU oracle (untuned, one thread) on the first tokens of the same
    workload: routing, each token's k experts forward and backward, the
    shared expert and the router backward.  Weight copies to the host are
    outside the timing."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle

    def host(t):
        return t.detach().float().cpu().numpy()

    k = cfg.k
    per_token = 18.0 * k * cfg.d * cfg.f + 18.0 * cfg.d * cfg.fs + 6.0 * cfg.d * cfg.E
    w_r = host(inp["w_r"])
    bias = None if inp["logit_bias"] is None else host(inp["logit_bias"])
    shared = (host(inp["ws13"]), host(inp["ws2"])) if cfg.fs else None
    spent, ntok = 0.0, 0
    with threadpool_limits(1):
        while spent < budget_s and ntok < 256:
            t = ntok
            x_t = host(inp["x"][t:t + 1]).astype(np.float64)
            dout_t = host(inp["dout"][t]).astype(np.float64)
            c0 = time.perf_counter()
            z = oracle.router_logits(x_t, w_r, bias)
            r = oracle.route(z, k, cfg.score, cfg.renorm)
            spent += time.perf_counter() - c0
            dw = np.zeros((1, k))
            for j in range(k):
                e = int(r["topk_idx"][0, j])
                w13e, w2e = host(inp["w13"][e]), host(inp["w2"][e])
                c0 = time.perf_counter()
                a, b, h, y = oracle.expert_ffn(x_t[0], w13e, w2e)
                dw[0, j] = dout_t @ y
                oracle.expert_ffn_bwd(x_t[0], w13e, w2e, a, b, h, r["topk_w"][0, j] * dout_t)
                spent += time.perf_counter() - c0
            c0 = time.perf_counter()
            if shared is not None:
                a, b, h, y = oracle.expert_ffn(x_t[0], *shared)
                oracle.expert_ffn_bwd(x_t[0], shared[0], shared[1], a, b, h, dout_t)
            dz = oracle.route_bwd(z, r["topk_idx"], r["topk_w"], dw, cfg.score, cfg.renorm)
            oracle.router_logits_bwd(x_t, w_r, dz)
            spent += time.perf_counter() - c0
            ntok += 1
    avail, model = cpu_identity()
    return {
        "value": per_token * ntok / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "cores_available": avail,
        "cpu_model": model,
        "kind": "oracle",
        "sample": (f"first {ntok} tokens of the {cfg.name} layer through the oracle's per-token "
                   f"loop (routing, {ntok * k} token-expert SwiGLU forward+backward pairs, shared "
                   f"expert, router backward), float64 NumPy, 1 thread, {spent:.1f} s; same "
                   f"algorithmic FLOPs per token as the GPU line"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU hot path only: the library runs on one GPU "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from routing_grouped_gemm_router_amd import inputs
    from routing_grouped_gemm_router_amd.layer import EventTimer, MoELayer

    if args.copy_calibration:
        n = args.copy_calibration // 16 * 16
        src = torch.empty(n, dtype=torch.uint8, device="cuda").view(torch.int32).fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return 0

    cfg = inputs.CONFIGS[args.config]
    if args.vendor_grouped_mm:
        if cfg.gemm != "bf16":
            print(f"{cfg.name}: the vendor comparison runs the bf16 layers", file=sys.stderr)
            return 2
        print(json.dumps(vendor_grouped_mm(cfg, args.seed)), flush=True)
        return 0
    if cfg.gemm not in ("bf16", "fp8", "mxfp8"):
        print(f"{cfg.name}: bench.py times the bf16, fp8 and mxfp8 expert paths", file=sys.stderr)
        return 2
    gemm_peak = PEAK_FP8_TFLOPS if cfg.gemm in ("fp8", "mxfp8") else PEAK_BF16_TFLOPS
    dev = "cuda"
    inp = inputs.layer_inputs(cfg, args.seed, dev)
    layer = MoELayer(cfg, inp, dev, recompute_act=args.recompute_act,
                     gate_in_ffn=args.gate_in_ffn)
    x, dout = inp["x"], inp["dout"]
    for _ in range(args.warmup):
        layer.forward(x)
        layer.backward(dout)
    torch.cuda.synchronize()

    timer = EventTimer()
    layer.timer = timer
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(x)
        layer.backward(dout)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    layer.timer = None
    ms_step = (t1 - t0) * 1e3 / args.steps

    spans = timer.summary()
    counts = layer.counts.cpu()
    n_nonempty = int((counts > 0).sum())
    n_rows = int(counts.sum())  # (token, slot) pairs with a row: T * k unless dropped
    work = kernel_work(cfg, n_nonempty, gated=args.gate_in_ffn, n_rows=n_rows,
                       sparse_router_bwd=layer.sparse_dz)
    kernels = {}
    for name, (ms, n) in spans.items():
        fl, by = work[name]
        kernels[name] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 2) if fl else None,
                         "GB/s": round(by / ms / 1e6, 1), "alg_bytes": int(by), "alg_flops": fl}
        tr = traffic_for(cfg.name, name)
        if tr is not None:  # counter-measured HBM bytes of this call
            kernels[name]["traffic"] = tr
            kernels[name]["traffic_GB/s"] = round(tr / ms / 1e6, 1)
    total_flops = sum(fl for fl, _ in work.values())
    value = total_flops / (ms_step / 1e3) / 1e12

    gemm_names = [n for n in kernels if "gemm" in n]
    gemm_ms = sum(kernels[n]["ms"] for n in gemm_names)
    gemm_flops = sum(work[n][0] for n in gemm_names)
    pc_names = [n for n in ("permute", "combine", "combine_bwd", "permute_bwd") if n in kernels]
    pc_ms = sum(kernels[n]["ms"] for n in pc_names)
    pc_bytes = sum(work[n][1] for n in pc_names)
    pc_tr = [kernels[n].get("traffic") for n in pc_names]
    pc_traffic = sum(pc_tr) if pc_tr and None not in pc_tr else None

    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    fl, by = work[dom]
    ms = kernels[dom]["ms"]
    ridge = gemm_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if fl and "gemm" in dom and fl / by >= ridge:
        roof = {"bound": "mfma", "achieved": round(fl / ms / 1e9, 1), "peak": gemm_peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["alg_flops_per_launch"] = fl
    roof["alg_bytes_per_launch"] = int(by)
    roof["ms_per_launch"] = ms
    roof["traffic"] = traffic_for(cfg.name, dom)

    router = [n for n in ("router_logits", "router_logits_bwd") if n in kernels]
    router_ms = sum(kernels[n]["ms"] for n in router)
    router_fl = sum(work[n][0] for n in router)
    cold = cold_dirty = None
    if args.cold_reps > 0:
        cold = cold_data_movement(layer, dout, work, args.cold_reps, clean=True)
        cold_dirty = cold_data_movement(layer, dout, work, args.cold_reps, clean=False)["total"]

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.gemm,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, generated on the GPU)",
        "config": {"workload": cfg.name, "routing": cfg.routing,
                   "expert_bias": cfg.expert_bias_std > 0,
                   "recompute_act": bool(args.recompute_act), "gate_in_ffn": bool(args.gate_in_ffn),
                   "router_bwd": "chosen experts" if layer.sparse_dz else "dense",
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "ffn": cfg.f, "shared_ffn": cfg.fs, "score": cfg.score, "renorm": cfg.renorm,
                   "router_bias": cfg.bias, "experts_with_rows": n_nonempty,
                   "routed_rows": n_rows,
                   "max_rows_per_expert": int(counts.max())},
        "grouped_gemm": {"TFLOP/s": round(gemm_flops / gemm_ms / 1e9, 1),
                         "frac_peak": round(gemm_flops / gemm_ms / 1e9 / gemm_peak, 4),
                         "peak": gemm_peak,
                         "ms": round(gemm_ms, 3)},
        "permute_combine": {"GB/s": round(pc_bytes / pc_ms / 1e6, 1),
                            "frac_hbm_peak": round(pc_bytes / pc_ms / 1e6 / PEAK_HBM_GBS, 4),
                            "ms": round(pc_ms, 4),
                            "traffic": pc_traffic,
                            "traffic_GB/s": (round(pc_traffic / pc_ms / 1e6, 1)
                                             if pc_traffic is not None else None),
                            "cold": cold, "cold_after_dirty_flush": cold_dirty},
        "router": {"TFLOP/s": round(router_fl / router_ms / 1e9, 1) if router_ms else None,
                   "frac_peak": (round(router_fl / router_ms / 1e9 / PEAK_F32_TFLOPS, 4)
                                 if router_ms else None),
                   "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s", "ms": round(router_ms, 4),
                   "engine": "fp32 vector ALUs"},
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
