"""Seeded synthetic inputs for the MoE layer.

This module holds only random-number generation and the shapes of the
workloads; none of the layer's arithmetic.  Both the HIP path and the CPU
reference take their inputs from here.

Workloads (shapes of the models the Megatron Core MoE report trains, section 8
"Performance Evaluation" and the upcycling abstract on the same author page;
all tensors synthetic, N(0, 1) activations and N(0, 1/fan_in) weights):

  tiny_fp32          T=64    d=128  E=4   k=2 f=256   fp32, softmax top-2, renorm
  llama3_8b_e8k2     T=8192  d=4096 E=8   k=2 f=14336 bf16, softmax top-2, renorm
  qwen3_235b_e128k8  T=16384 d=4096 E=128 k=8 f=1536  bf16, softmax top-8, renorm,
                     logit bias -ln(rank) over a seeded expert permutation (Zipf s=1)
  deepseek_v3_e256k8 T=8192  d=7168 E=256 k=8 f=2048  bf16, sigmoid top-8, renorm,
                     logit bias N(0, variance 0.5), one shared expert fs=2048
  deepseek_v3_fp8    as deepseek_v3_e256k8 with T=32768 and fp8 E4M3 expert GEMMs
  deepseek_v3_mxfp8  as deepseek_v3_fp8 with MXFP8 expert GEMMs (1 x 32 blocks,
                     E8M0 scales)
  deepseek_v3_balanced as deepseek_v3_e256k8 with force-balanced routing (the
                     benchmark setting of section 8: every expert gets exactly
                     T*k/E rows), replayed from a seeded assignment
  small_balanced     T=512 d=256 E=16 k=4 f=256 shared 128, bf16, force-balanced
  deepseek_v3_capacity as deepseek_v3_e256k8 with capacity-limited dropping
                     (capacity factor 1.0: at most T*k/E rows per expert)
  small_capacity     T=513 d=128 E=16 k=4 f=128, Zipf-biased softmax routing,
                     capacity factor 1.25
  small_pad_to_max   small_capacity with every expert's segment padded to the
                     capacity (static offsets e * C)
  deepseek_v3_pad_to_max deepseek_v3_capacity padded to the capacity
  small_aux          T=300 d=256 E=8 k=2 f=256 shared 128, sigmoid routing with
                     an auxiliary load-balancing loss (coefficient 0.01)
  deepseek_v3_expert_bias as deepseek_v3_e256k8 with the selection-only expert
                     bias (auxiliary-loss-free balancing) instead of the logit
                     bias: N(0, 0.01^2) initial bias, update rate 1e-3
  small_expert_bias  T=512 d=256 E=16 k=4 f=256 shared 128, sigmoid scores with
                     an N(0, 0.05^2) selection bias, update rate 1e-3

Generation: each tensor (and each expert's slice of a weight) is drawn from
its own torch generator seeded from (seed, stream id), as float32 normals
scaled by the standard deviation and rounded to the storage dtype (bf16 by
round-to-nearest-even).  Large workloads are drawn directly on the GPU.
"""

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    fs: int = 0                 # shared-expert ffn width, 0 = none
    dtype: str = "bf16"         # storage dtype of activations / expert weights
    gemm: str = "bf16"          # arithmetic of the expert GEMMs: f32 | bf16 | fp8 | mxfp8
    score: str = "softmax"      # softmax | sigmoid
    renorm: bool = True
    bias: str = "none"          # none | zipf | normal
    bias_var: float = 0.5
    zipf_s: float = 1.0
    routing: str = "topk"       # topk | balanced (experts given, replayed)
    capacity_factor: float = 0.0  # > 0: each expert keeps ceil(factor*T*k/E) rows
    pad_to_max: bool = False      # with a capacity: every expert's segment padded to it
    aux_loss_coeff: float = 0.0   # > 0: auxiliary load-balancing loss
    # > 0: selection-only expert bias on sigmoid scores (auxiliary-loss-free
    # balancing), drawn N(0, std^2), moved by the update rate after each route
    expert_bias_std: float = 0.0
    expert_bias_rate: float = 0.0
    note: str = field(default="", compare=False)

    @property
    def N(self):
        return self.T * self.k

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


CONFIGS = {
    "tiny_fp32": LayerConfig("tiny_fp32", T=64, d=128, E=4, k=2, f=256, dtype="f32", gemm="f32"),
    "llama3_8b_e8k2": LayerConfig("llama3_8b_e8k2", T=8192, d=4096, E=8, k=2, f=14336),
    "qwen3_235b_e128k8": LayerConfig("qwen3_235b_e128k8", T=16384, d=4096, E=128, k=8, f=1536,
                                     bias="zipf"),
    "deepseek_v3_e256k8": LayerConfig("deepseek_v3_e256k8", T=8192, d=7168, E=256, k=8, f=2048,
                                      fs=2048, score="sigmoid", bias="normal"),
    "deepseek_v3_fp8": LayerConfig("deepseek_v3_fp8", T=32768, d=7168, E=256, k=8, f=2048,
                                   fs=2048, gemm="fp8", score="sigmoid", bias="normal"),
    "deepseek_v3_mxfp8": LayerConfig("deepseek_v3_mxfp8", T=32768, d=7168, E=256, k=8, f=2048,
                                     fs=2048, gemm="mxfp8", score="sigmoid", bias="normal"),
    "deepseek_v3_balanced": LayerConfig("deepseek_v3_balanced", T=8192, d=7168, E=256, k=8,
                                        f=2048, fs=2048, score="sigmoid", bias="normal",
                                        routing="balanced"),
    "small_balanced": LayerConfig("small_balanced", T=512, d=256, E=16, k=4, f=256, fs=128,
                                  score="sigmoid", bias="normal", routing="balanced"),
    "deepseek_v3_capacity": LayerConfig("deepseek_v3_capacity", T=8192, d=7168, E=256, k=8,
                                        f=2048, fs=2048, score="sigmoid", bias="normal",
                                        capacity_factor=1.0),
    "small_capacity": LayerConfig("small_capacity", T=513, d=128, E=16, k=4, f=128, bias="zipf",
                                  capacity_factor=1.25),
    "deepseek_v3_expert_bias": LayerConfig("deepseek_v3_expert_bias", T=8192, d=7168, E=256, k=8,
                                           f=2048, fs=2048, score="sigmoid", expert_bias_std=0.01,
                                           expert_bias_rate=1e-3),
    "small_expert_bias": LayerConfig("small_expert_bias", T=512, d=256, E=16, k=4, f=256, fs=128,
                                     score="sigmoid", expert_bias_std=0.05, expert_bias_rate=1e-3),
    "small_pad_to_max": LayerConfig("small_pad_to_max", T=513, d=128, E=16, k=4, f=128,
                                    bias="zipf", capacity_factor=1.25, pad_to_max=True),
    "deepseek_v3_pad_to_max": LayerConfig("deepseek_v3_pad_to_max", T=8192, d=7168, E=256, k=8,
                                          f=2048, fs=2048, score="sigmoid", bias="normal",
                                          capacity_factor=1.0, pad_to_max=True),
    "small_aux": LayerConfig("small_aux", T=300, d=256, E=8, k=2, f=256, fs=128, score="sigmoid",
                             bias="normal", aux_loss_coeff=0.01),
}

# stream ids: one per tensor; expert weights add the expert index
_S_X, _S_WR, _S_BIAS, _S_DOUT, _S_SHARED, _S_ROUTE, _S_EBIAS = 1, 2, 3, 4, 5, 6, 8
_S_W1, _S_W3, _S_W2 = 1 << 20, 2 << 20, 3 << 20


def balanced_experts(T, E, k, seed, device="cpu"):
    """A forced assignment in which every expert gets exactly T*k/E (token,
    slot) pairs (T*k divisible by E, k <= E): with a seeded permutation pi of
    the tokens, slot j of token t goes to expert (pi(t)*k + j) mod E, so a
    token's k experts are k consecutive experts (distinct) and the pairs cycle
    through all experts evenly.  int32 [T, k]."""
    assert k <= E and (T * k) % E == 0
    pi = torch.randperm(T, generator=generator(seed, _S_ROUTE, "cpu"))
    idx = (pi[:, None] * k + torch.arange(k)[None, :]) % E
    return idx.to(torch.int32).to(device)


def generator(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & ((1 << 63) - 1))
    return g


def normal(shape, std, seed, stream, device, dtype):
    """float32 N(0, std^2) rounded to ``dtype``."""
    g = generator(seed, stream, device)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def logit_bias(cfg, seed, device="cpu"):
    """Per-expert constant added to the router logits (fp32) or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "zipf":
        g = generator(seed, _S_BIAS, "cpu")
        perm = torch.randperm(cfg.E, generator=g)          # seeded expert order
        rank = (perm + 1).to(torch.float64)
        return (-cfg.zipf_s * torch.log(rank)).to(torch.float32).to(device)
    if cfg.bias == "normal":
        return normal((cfg.E,), math.sqrt(cfg.bias_var), seed, _S_BIAS, device, torch.float32)
    raise ValueError(cfg.bias)


def expert_weights(cfg, seed, device, E=None, f=None, stream_base=0):
    """W13 [E, d, 2f] = [W1 | W3] and W2 [E, f, d], one expert at a time."""
    E = cfg.E if E is None else E
    f = cfg.f if f is None else f
    dt = cfg.torch_dtype()
    w13 = torch.empty((E, cfg.d, 2 * f), dtype=dt, device=device)
    w2 = torch.empty((E, f, cfg.d), dtype=dt, device=device)
    s1 = 1.0 / math.sqrt(cfg.d)
    s2 = 1.0 / math.sqrt(f)
    for e in range(E):
        w13[e, :, :f] = normal((cfg.d, f), s1, seed, stream_base + _S_W1 + e, device, dt)
        w13[e, :, f:] = normal((cfg.d, f), s1, seed, stream_base + _S_W3 + e, device, dt)
        w2[e] = normal((f, cfg.d), s2, seed, stream_base + _S_W2 + e, device, dt)
    return w13, w2


def layer_inputs(cfg, seed, device="cpu"):
    """All inputs of one layer pass, forward and backward."""
    dt = cfg.torch_dtype()
    inp = dict(
        x=normal((cfg.T, cfg.d), 1.0, seed, _S_X, device, dt),
        w_r=normal((cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d), seed, _S_WR, device, torch.float32),
        logit_bias=logit_bias(cfg, seed, device),
        dout=normal((cfg.T, cfg.d), 1.0, seed, _S_DOUT, device, dt),
    )
    inp["w13"], inp["w2"] = expert_weights(cfg, seed, device)
    if cfg.fs:
        ws13, ws2 = expert_weights(cfg, seed, device, E=1, f=cfg.fs, stream_base=_S_SHARED << 24)
        inp["ws13"], inp["ws2"] = ws13[0], ws2[0]
    if cfg.routing == "balanced":
        inp["topk_idx_in"] = balanced_experts(cfg.T, cfg.E, cfg.k, seed, device)
    if cfg.expert_bias_std > 0:
        inp["expert_bias"] = normal((cfg.E,), cfg.expert_bias_std, seed, _S_EBIAS, device,
                                    torch.float32)
    return inp


def resample_rows(x, rows, seed, attempt):
    """Fresh N(0, 1) rows for the given token indices (in place)."""
    for t in rows:
        x[t] = normal((x.shape[1],), 1.0, seed, (7 << 28) + attempt * 1_000_000 + int(t),
                      x.device, x.dtype)
    return x


def random_segments(M, G, seed, empty_frac=0.0, skew=0.0):
    """Seeded partition of M rows into G contiguous segments (int64 offsets
    [G+1]); some segments may be empty.  Used to drive the grouped GEMM with
    ragged, adversarial group sizes."""
    g = generator(seed, 99, "cpu")
    w = torch.rand(G, generator=g, dtype=torch.float64) + 1e-3
    if skew:
        w = w ** (1.0 + skew * 8)
    if empty_frac:
        w[torch.rand(G, generator=g, dtype=torch.float64) < empty_frac] = 0.0
    if float(w.sum()) == 0:
        w[0] = 1.0
    cuts = torch.floor(torch.cumsum(w, 0) / w.sum() * M).to(torch.int64)
    cuts[-1] = M
    offsets = torch.zeros(G + 1, dtype=torch.int64)
    offsets[1:] = cuts
    return offsets
