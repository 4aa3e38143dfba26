"""Oracle-side decoding of stored inputs to fp64 (test infrastructure).

Pinned by tests/test_oracle_num.py: all 65,536 bf16 patterns against
torch's bfloat16 type, and hand-worked values of the format.
"""
import numpy as np


def f64(a) -> np.ndarray:
    """Exact fp64 value of a stored array: float32/float16/float64 as is,
    uint16 as bf16 bit patterns (bf16 is the upper half of an fp32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
