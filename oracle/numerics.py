"""Bit-pattern decoders for the 16-bit formats the layer's inputs use.

bf16 is the top half of an IEEE binary32; fp16 is IEEE binary16.  Both widen
exactly to fp64.
"""

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 IEEE binary16 bit patterns -> exact fp64 values."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
