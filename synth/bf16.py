"""bf16 <-> fp32 bit-pattern conversion for seeded inputs (numpy only).

Weights and synthetic KV are produced in fp32, rounded once to bf16 with
round-to-nearest-even, and handed to both sides as the same 16-bit
patterns.  The oracle widens those patterns back to fp32/fp64 exactly.
"""

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((b + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen uint16 bf16 patterns to fp32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)
