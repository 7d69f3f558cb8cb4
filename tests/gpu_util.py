"""Helpers shared by the GPU parity tests (tolerances, conversions, input
construction that needs the oracle)."""
import numpy as np
import torch

import oracle
from routing_grouped_gemm_router_amd import inputs

# max|err| / max|ref| bounds per arithmetic type (the layer's stated tolerances)
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "mxfp8": 6e-2}


def np64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_err(got, ref):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    print(f"  {name}: max|err|/max|ref| = {e:.3e} (bound {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:.1e}"
    return e


def boundary_gaps(z, k):
    """Per token: gap between the k-th and (k+1)-th largest key (inf if k = E)."""
    s = -np.sort(-np.asarray(z, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def near_tie_tokens(z, k, rel_gap):
    """Tokens whose selection or slot order an fp32 rounding difference could
    change: two of the top k+1 keys (by the oracle) closer than
    rel_gap * (1 + |key|)."""
    s = -np.sort(-np.asarray(z, np.float64), axis=1)[:, :k + 1]
    if s.shape[1] < 2:
        return np.zeros(0, dtype=np.int64)
    gaps = s[:, :-1] - s[:, 1:]
    close = gaps < rel_gap * (1.0 + np.abs(s[:, :-1]))
    return np.nonzero(close.any(axis=1))[0]


def layer_inputs_without_near_ties(cfg, seed, device="cpu", rel_gap=1e-4, attempts=20):
    """Seeded layer inputs whose routing is not decided by fp32 rounding: a
    token with two of its top k+1 keys (by the oracle) closer than
    rel_gap * (1 + |key|) gets a fresh x row, so the GPU's fp32 router (a
    different summation order) must select the same experts in the same slot
    order.  With a selection-only expert bias the keys are
    sigmoid(z) + bias."""
    inp = inputs.layer_inputs(cfg, seed, device)
    sel = inp.get("expert_bias")
    bias = None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy()
    w_r = inp["w_r"].cpu().numpy()
    for attempt in range(attempts):
        x = inp["x"].cpu()
        z = oracle.router_logits(np64(x), w_r, bias)
        if sel is not None:
            z = oracle.selection_keys(z, sel.cpu().numpy())
        bad = near_tie_tokens(z, cfg.k, rel_gap)
        if len(bad) == 0:
            return inp
        inputs.resample_rows(inp["x"], [int(t) for t in bad], seed, attempt)
    raise RuntimeError("could not draw inputs without near-ties")
