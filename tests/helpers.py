"""Shared test helpers: tolerance metric, device transfer, oracle-side input preparation."""
import numpy as np

import workloads

# Gate: max|gpu - ref| / max|ref| over the whole tensor.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype=None, device="cuda:0"):
    """numpy float32 -> device tensor; bf16 arrays must already hold bf16 values."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def host(t):
    return t.float().cpu().numpy()


def store_like(x64, dtype: str):
    """fp64 oracle-side operand -> the stored dtype's values (float32 array)."""
    x = np.asarray(x64, dtype=np.float32)
    return workloads.round_bf16(x) if dtype == "bf16" else x
