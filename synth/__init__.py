"""Seeded synthetic inputs shared by the oracle and the HIP path.

This package holds input generation only: model dimensions, seeded weight
tensors (as bf16 bit patterns), token ids, the page allocator and the
batch layouts of the benchmark workloads.  It contains none of the
arithmetic of the forward step; both the oracle (``oracle/``) and the
product binding consume what it produces and neither depends on the other.
"""

from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32
from .model import ModelConfig, make_weights, layer_weight_names
from .hashfill import splitmix64_fill
from .workloads import (
    Item, Batch, PageAllocator, EMBED, PREFILL, DECODE,
    POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST,
)

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "ModelConfig", "make_weights",
    "layer_weight_names", "splitmix64_fill", "Item", "Batch", "PageAllocator",
    "EMBED", "PREFILL", "DECODE", "POOL_MEAN", "POOL_WMEAN", "POOL_CLS",
    "POOL_LAST",
]
