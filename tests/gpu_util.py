"""Helpers shared by the GPU parity tests (tolerances, conversions)."""
import numpy as np
import torch


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
