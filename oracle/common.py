"""Conversions shared by the oracle modules (test infrastructure only)."""
import numpy as np


def f64(x):
    """Exact float64 copy of a NumPy array or torch tensor (bf16/fp16/fp32/fp64)."""
    if hasattr(x, "detach"):
        t = x.detach().cpu()
        if t.is_floating_point():
            t = t.double()
        return t.numpy()
    a = np.asarray(x)
    if a.dtype.kind == "f":
        return a.astype(np.float64)
    return a


def i64(x):
    """int64 NumPy copy of an integer array or tensor."""
    if hasattr(x, "detach"):
        return x.detach().cpu().to(dtype=__import__("torch").int64).numpy()
    return np.asarray(x).astype(np.int64)
