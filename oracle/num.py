"""Oracle-side decoding of stored inputs to fp64 (test infrastructure)."""
import numpy as np


def f64(a) -> np.ndarray:
    """Exact fp64 value of a stored array: float32/float16/float64 as is,
    uint16 as bf16 bit patterns (bf16 is the upper half of an fp32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
