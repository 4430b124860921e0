"""Helpers for the GPU parity tests: upload seeded inputs, poison outputs, compare to the oracle."""

import numpy as np


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_device(t, device="cuda"):
    """Upload an inputs.Tensor bit-exactly."""
    import torch
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.bits)).to(device)
    raw = torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16))
    return raw.view(torch_dtype(t.dtype)).to(device)


def nan_like(shape, dtype, device="cuda"):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device=device)


def host64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values (unwritten or overflowed outputs)"
    return float(np.abs(got - ref).max()) if got.size else 0.0


def check(name, got, ref, tol, log=None):
    e = max_err(got, ref)
    if log is not None:
        log.append((name, e, tol))
    print(f"    {name}: max_abs_err={e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: max abs error {e:.3e} > {tol:g}"
    return e


# Tolerances against the float64 oracle, by input dtype (O / gradients, LSE).
TOL = {"f32": (1e-5, 1e-5), "f16": (2e-2, 1e-3), "bf16": (2e-2, 1e-3)}
