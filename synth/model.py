"""Model dimensions and seeded random-init weights (bf16 bit patterns).

Linear weights are stored [out_features, in_features], row-major, and drawn
from N(0, std) with a per-tensor numpy generator seeded from (seed, name).
Norm gains are 1 unless ``gain_std`` is set, in which case they are
1 + N(0, gain_std) (used by tests so that a dropped gain is visible).
"""

from dataclasses import dataclass, asdict, replace
import concurrent.futures as cf
import os
import zlib

import numpy as np

from .bf16 import f32_to_bf16_bits


@dataclass(frozen=True)
class ModelConfig:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    lora_rank: int = 0
    page_size: int = 16
    rope_theta: float = 1e4
    rms_eps: float = 1e-5
    lora_scale: float = 1.0
    dtype: str = "bf16"      # number format of weights, KV and compute: "bf16" or "f32"

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    def as_dict(self):
        return asdict(self)

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


# Tiny decoder of the small correctness workload: 2 layers, d 64, 4 q / 2 kv
# heads of 16, SwiGLU 176, theta 1e4, vocab 256, KV pages of 8 tokens.
TINY = ModelConfig(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                   ffn_dim=176, vocab=256, lora_rank=0, page_size=8, rope_theta=1e4)

# The same tiny decoder in fp32 (weights drawn in fp32, not rounded to bf16).
TINY_F32 = TINY.with_(dtype="f32")

# Mistral-7B shape: d 4096, 32 q / 8 kv heads of 128, SwiGLU 14336,
# theta 1e6, vocab 32768 (the public Mistral-7B vocabulary size).
MISTRAL_7B = ModelConfig(n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8,
                         head_dim=128, ffn_dim=14336, vocab=32768, lora_rank=16,
                         page_size=16, rope_theta=1e6)

# Llama-3.1-8B shape: as Mistral-7B but theta 5e5 and vocab 128256.
LLAMA31_8B = MISTRAL_7B.with_(rope_theta=5e5, vocab=128256)


def layer_weight_names():
    return ["w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_ffn",
            "lora_a_qkv", "lora_b_qkv", "lora_a_o", "lora_b_o"]


def weight_shapes(cfg: ModelConfig):
    """Shapes of every tensor: globals, then per-layer (same for all layers)."""
    r = cfg.lora_rank
    glob = {
        "tok_emb": (cfg.vocab, cfg.d_model),
        "lm_head": (cfg.vocab, cfg.d_model),
        "g_final": (cfg.d_model,),
    }
    layer = {
        "w_qkv": (cfg.qkv_dim, cfg.d_model),
        "w_o": (cfg.d_model, cfg.q_dim),
        "w_gate_up": (2 * cfg.ffn_dim, cfg.d_model),  # gate rows, then up rows
        "w_down": (cfg.d_model, cfg.ffn_dim),
        "g_attn": (cfg.d_model,),
        "g_ffn": (cfg.d_model,),
        "lora_a_qkv": (3 * r, cfg.d_model),   # q, k, v shrink rows
        "lora_b_qkv": (cfg.qkv_dim, r),       # expand, one row per output column
        "lora_a_o": (r, cfg.q_dim),
        "lora_b_o": (cfg.d_model, r),
    }
    return glob, layer


def _tensor_seed(seed: int, name: str) -> int:
    return (int(seed) * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFF


CHUNK = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _POOL


def normal_bf16(key, n: int, std: float, mean: float = 0.0) -> np.ndarray:
    """n values mean + N(0, std), rounded to bf16 bits.  Generated in chunks of
    2^22 values, chunk i from numpy's PCG64 seeded with (key..., i), so the
    result depends only on (key, n, std, mean)."""
    out = np.empty(n, np.uint16)
    key = list(key)

    def work(i):
        m = min(CHUNK, n - i * CHUNK)
        v = np.random.default_rng(key + [i]).standard_normal(m, dtype=np.float32)
        v *= np.float32(std)
        if mean:
            v += np.float32(mean)
        out[i * CHUNK: i * CHUNK + m] = f32_to_bf16_bits(v)

    list(_pool().map(work, range((n + CHUNK - 1) // CHUNK)))
    return out


def normal_f32(key, n: int, std: float, mean: float = 0.0) -> np.ndarray:
    """As normal_bf16 (same generator and chunking), kept in fp32."""
    out = np.empty(n, np.float32)
    key = list(key)
    for i in range((n + CHUNK - 1) // CHUNK):
        m = min(CHUNK, n - i * CHUNK)
        v = np.random.default_rng(key + [i]).standard_normal(m, dtype=np.float32)
        v *= np.float32(std)
        if mean:
            v += np.float32(mean)
        out[i * CHUNK: i * CHUNK + m] = v
    return out


def make_tensor(seed: int, name: str, shape, std: float = 0.02,
                gain_std: float = 0.0, f32: bool = False) -> np.ndarray:
    """One seeded tensor as uint16 bf16 bits (float32 values with f32)."""
    n = int(np.prod(shape)) if len(shape) else 1
    key = [_tensor_seed(seed, name)]
    base = name.split(".")[-1]
    if base.startswith("g_"):
        if not gain_std:
            ones = np.ones(shape, np.float32)
            return ones if f32 else f32_to_bf16_bits(ones)
        if f32:
            return normal_f32(key, n, gain_std, mean=1.0).reshape(shape)
        return normal_bf16(key, n, gain_std, mean=1.0).reshape(shape)
    if f32:
        return normal_f32(key, n, std).reshape(shape)
    return normal_bf16(key, n, std).reshape(shape)


def make_weights(cfg: ModelConfig, seed: int = 0, std: float = 0.02,
                 gain_std: float = 0.0, zero_lora_b: bool = False):
    """All weights as {name: uint16 bf16 bits}, or {name: float32} for a
    model of dtype "f32"; layer tensors named 'layers.<l>.<n>'."""
    glob, layer = weight_shapes(cfg)
    f32 = cfg.dtype == "f32"
    zdt = np.float32 if f32 else np.uint16
    w = {}
    for n, s in glob.items():
        w[n] = make_tensor(seed, n, s, std, gain_std, f32)
    for l in range(cfg.n_layers):
        for n, s in layer.items():
            full = f"layers.{l}.{n}"
            if n.startswith("lora_") and cfg.lora_rank == 0:
                w[full] = np.zeros(s, zdt)
            elif n.startswith("lora_b") and zero_lora_b:
                w[full] = np.zeros(s, zdt)
            else:
                w[full] = make_tensor(seed, full, s, std, gain_std, f32)
    return w
