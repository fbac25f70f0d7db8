"""bfloat16 encoding of float32 arrays (input encoding only).

bfloat16 keeps the upper 16 bits of an IEEE-754 binary32 value. Rounding from
float32 is round-to-nearest, ties-to-even on the 16 discarded bits. The
workloads hold no NaN or infinity, so no special case is needed for them.
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen uint16 bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
