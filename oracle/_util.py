"""Exact conversion of inputs to fp64 arrays (oracle helper)."""
import numpy as np


def f64(x) -> np.ndarray:
    """Return x as an fp64 numpy array; bf16/fp16/fp32 values upcast exactly."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if x.dtype.is_floating_point and x.dtype.itemsize < 8:
            x = x.float()
        x = x.double().numpy() if x.dtype.is_floating_point else x.numpy()
    return np.asarray(x, dtype=np.float64)
