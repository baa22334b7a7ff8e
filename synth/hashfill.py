"""Counter-based synthetic values: SplitMix64 (Steele, Lea and Flood, 2014).

Value ``i`` of tensor ``tensor_id`` under ``seed`` is

    z  = ((seed << 32) ^ tensor_id) + (i + 1) * 0x9E3779B97F4A7C15   (mod 2^64)
    z  = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
    z  = (z ^ (z >> 27)) * 0x94D049BB133111EB
    h  =  z ^ (z >> 31)
    u  = (h >> 40) * 2^-24                     in [0, 1), exact in fp32
    v  = bf16_rne(fp32((2u - 1) * 1.7320508f))  zero mean, unit variance

Every step is exact integer arithmetic or a single correctly rounded fp32
operation, so any implementation of this definition yields the same bits.
"""

import numpy as np

from .bf16 import f32_to_bf16_bits

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SQRT3_F32 = np.float32(1.7320508)


def splitmix64_fill(seed: int, tensor_id: int, n: int, start: int = 0) -> np.ndarray:
    """Return uint16 bf16 bit patterns for indices [start, start+n)."""
    key = np.uint64(((int(seed) & 0xFFFFFFFF) << 32) ^ (int(tensor_id) & 0xFFFFFFFF))
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    u = (z >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    t = np.float32(2.0) * u - np.float32(1.0)
    return f32_to_bf16_bits(t * SQRT3_F32)
