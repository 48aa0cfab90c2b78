"""Exact widening of stored values to fp64 (oracle; test infrastructure only).

The oracle reads exactly the values that are stored in device memory.  A bf16
value is the top half of an IEEE fp32 word, so shifting its 16 bits into the
high half of a 32-bit word and reinterpreting gives the fp32 number exactly;
widening fp32 to fp64 is exact as well.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> fp64 array, exactly."""
    u16 = np.asarray(bits)
    if u16.dtype != np.uint16:
        raise TypeError("bf16 values must be given as uint16 bit patterns")
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(x, dtype):
    """Stored array in ``dtype`` ('bf16' bit patterns or 'f32') -> fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        a = np.asarray(x)
        if a.dtype != np.float32:
            raise TypeError("f32 values must be given as float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")
