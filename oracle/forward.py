"""One heterogeneous-batch forward step, written as the plain definition.

"Efficient Iterative Retrieval with Heterogeneous Batching" (paperpeel full
text): §3.1 High-Level Workflow — forward applies the same attention and
feed-forward layers to every request type, which differ only in input
length, then emit diverges (next-token logits for generation, incremental
pooling for embedding); §3.2 Batch Unit — embedding chunks, generation
prefill chunks and single-token decode rows share one pass; §2.2
(Generation) — a decode step reads the KV cache of earlier tokens and
appends its own; §2.2 (Parameter sharing) and §5.1 — the embedding model is
the shared backbone plus a LoRA adapter.  Summary page (agihunt): one pass
runs attention and FFN once over all three batch units.

The model is a pre-norm decoder: RMSNorm, q/k/v projections with
rotate-half RoPE, causal attention with grouped KV heads, output projection
and residual, RMSNorm, SwiGLU feed-forward and residual; a final RMSNorm
feeds both the LM head and the pooler.  The pages name only the models
(Mistral-7B, LLaMA3.1-8B), so these internals are the public architecture
of those models (no biases, no sliding window, untied embeddings).

Readings: the LoRA delta s * (h A^T) B^T is added to q, k, v and to the
output projection for embedding rows only, including the K/V that those
rows write to the cache; chunk k of a request attends to the KV of chunks
1..k-1 (required for chunked pooling to equal a single pass); a decode row
with context c sits at position c and attends to positions 0..c.

Everything is computed per request: an item's rows read and write only its
own pages, so any sub-batch of items gives the same result for those items.
"""

from dataclasses import dataclass

import numpy as np

from synth.bf16 import bf16_bits_to_f32
from .pack import pack_py, Limits, EMBED, PREFILL, DECODE
from .pooling import pool_item


def widen_weights(bits: dict, dtype=np.float32) -> dict:
    """bf16 bit patterns -> float arrays of ``dtype`` (exact widening); fp32
    arrays (an fp32 model's weights) are taken as they are."""
    return {k: (v.astype(dtype) if v.dtype == np.float32 else bf16_bits_to_f32(v).astype(dtype))
            for k, v in bits.items()}


def new_pool(n_slots: int, d: int, dtype=np.float32, buf_rows: int = 0) -> dict:
    """Pooling state; ``buf_rows`` > 0 adds the BUFFER kind's hidden-state
    buffer [n_slots, buf_rows, d]."""
    p = {"sum": np.zeros((n_slots, d), dtype), "wsum": np.zeros(n_slots, dtype),
         "kept": np.zeros((n_slots, d), dtype)}
    if buf_rows:
        p["buf"] = np.zeros((n_slots, buf_rows, d), dtype)
    return p


def new_kv(cfg, n_pages: int, dtype=np.float32, k_bits=None, v_bits=None):
    """Per-layer K and V pools [n_pages, n_kv_heads, page_size, head_dim]."""
    shape = (n_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)
    K, V = [], []
    for l in range(cfg.n_layers):
        if k_bits is None:
            K.append(np.zeros(shape, dtype))
            V.append(np.zeros(shape, dtype))
        else:
            K.append(bf16_bits_to_f32(k_bits[l]).astype(dtype))
            V.append(bf16_bits_to_f32(v_bits[l]).astype(dtype))
    return K, V


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, pos, theta):
    """Rotate-half rotary embedding of x [T, H, hd] at integer positions pos [T].

    Pair i (i < hd/2) is (x[i], x[i + hd/2]) rotated by pos * theta^(-2i/hd).
    Angles are formed in fp64 whatever the working precision.
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = np.float64(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(x.dtype)[:, None, :]
    sin = np.sin(ang).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attend_item(q, K, V, ctx):
    """Causal attention of one item.

    q [n, Hq, hd] holds the item's rows at positions ctx..ctx+n-1; K, V
    [ctx+n, Hkv, hd] hold keys/values at positions 0..ctx+n-1.  Row j sees
    positions 0..ctx+j.  Query head h reads KV head h // (Hq / Hkv).
    Softmax subtracts the row maximum before exponentiating.
    """
    n, Hq, hd = q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    L = K.shape[0]
    visible = np.arange(L)[None, :] <= (ctx + np.arange(n))[:, None]
    out = np.zeros_like(q)
    scale = 1.0 / np.sqrt(hd)
    for h in range(Hq):
        g = h // grp
        s = (q[:, h, :] @ K[:, g, :].T) * q.dtype.type(scale)
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out


def _gather_ctx(pool_l, pages, ps, length):
    p = np.arange(length)
    return pool_l[pages[p // ps], :, p % ps, :]


def _lora(h, A, B, s):
    return s * ((h @ A.T) @ B.T)


@dataclass
class StepOut:
    logits: np.ndarray       # [G, V]
    logit_req: np.ndarray    # [G]
    emb: np.ndarray          # [n_emb, d]
    emb_req: np.ndarray      # [n_emb]
    hidden: np.ndarray       # [T, d] residual stream after the last layer
    final: np.ndarray        # [T, d] final-norm output (LM-head / pooler input)
    meta: dict


def layer(cfg, W, l, x, batch, meta, kv, dtype=np.float32, trace=None):
    """Decoder layer ``l`` applied to the residual stream ``x`` [T, d] of
    ``batch`` (packing ``meta`` from ``pack_py``); appends every row's K/V to
    ``kv`` and returns the new residual stream.

    ``trace``, when a dict, receives this layer's intermediate values (for
    pins of single parts): ``qkv`` (the projections before RoPE, LoRA
    included), ``o`` (attention output [T, Hq*hd]), ``x_attn`` (residual
    after the attention block), ``h2`` (the FFN's normalised input) and
    ``act`` (silu(gate) * up).
    """
    K, V = kv
    T = batch.n_tokens
    Hq, Hkv, hd, F = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim
    r, s = cfg.lora_rank, dtype(cfg.lora_scale)
    qd, kd = cfg.q_dim, cfg.kv_dim
    ps = cfg.page_size
    TE = meta["n_embed_rows"]
    cu, pos = meta["cu_q"], meta["pos"]
    p = f"layers.{l}."
    h = rmsnorm(x, W[p + "g_attn"], dtype(cfg.rms_eps))
    qkv = h @ W[p + "w_qkv"].T
    if r > 0 and TE > 0:
        A, B = W[p + "lora_a_qkv"], W[p + "lora_b_qkv"]
        he = h[:TE]
        qkv[:TE, :qd] += _lora(he, A[:r], B[:qd], s)
        qkv[:TE, qd:qd + kd] += _lora(he, A[r:2 * r], B[qd:qd + kd], s)
        qkv[:TE, qd + kd:] += _lora(he, A[2 * r:], B[qd + kd:], s)
    q = rope(qkv[:, :qd].reshape(T, Hq, hd), pos, cfg.rope_theta)
    k = rope(qkv[:, qd:qd + kd].reshape(T, Hkv, hd), pos, cfg.rope_theta)
    v = qkv[:, qd + kd:].reshape(T, Hkv, hd)
    for i, it in enumerate(batch.items):
        pages = batch.item_pages(i)
        for j in range(it.n_tokens):
            pp = it.ctx_len + j
            K[l][pages[pp // ps], :, pp % ps, :] = k[cu[i] + j]
            V[l][pages[pp // ps], :, pp % ps, :] = v[cu[i] + j]
    o = np.zeros((T, Hq, hd), dtype)
    for i, it in enumerate(batch.items):
        pages = batch.item_pages(i)
        L = it.ctx_len + it.n_tokens
        Kc = _gather_ctx(K[l], pages, ps, L)
        Vc = _gather_ctx(V[l], pages, ps, L)
        o[cu[i]:cu[i + 1]] = attend_item(q[cu[i]:cu[i + 1]], Kc, Vc, it.ctx_len)
    o = o.reshape(T, qd)
    delta = o @ W[p + "w_o"].T
    if r > 0 and TE > 0:
        delta[:TE] += _lora(o[:TE], W[p + "lora_a_o"], W[p + "lora_b_o"], s)
    x = x + delta
    h2 = rmsnorm(x, W[p + "g_ffn"], dtype(cfg.rms_eps))
    gu = h2 @ W[p + "w_gate_up"].T
    a = silu(gu[:, :F]) * gu[:, F:]
    if trace is not None:
        trace.update(qkv=qkv, o=o, x_attn=x, h2=h2, act=a)
    return x + a @ W[p + "w_down"].T


def step(cfg, W, batch, kv, pool, dtype=np.float32, limits=None, trace=None):
    """Run one forward step of ``batch``; update ``kv`` and ``pool`` in place.

    W: widened weights (see ``widen_weights``), kv: (K, V) lists per layer.
    ``trace``, when a list, receives one dict per layer (see ``layer``) with
    the layer's input residual stream under ``x_in``.
    """
    K, V = kv
    if limits is None:
        limits = Limits(n_pages=K[0].shape[0] if K else 0, max_tokens=1 << 30,
                        max_items=1 << 30, max_pool_slots=pool["sum"].shape[0])
    meta = pack_py(cfg, batch, limits)
    d = cfg.d_model
    cu = meta["cu_q"]

    x = W["tok_emb"][batch.token_ids].astype(dtype)
    for l in range(cfg.n_layers):
        t = None
        if trace is not None:
            t = {"x_in": x}
            trace.append(t)
        x = layer(cfg, W, l, x, batch, meta, kv, dtype, trace=t)
    hf = rmsnorm(x, W["g_final"], dtype(cfg.rms_eps))
    lr = meta["logit_rows"]
    logits = hf[lr] @ W["lm_head"].T
    logit_req = np.array([batch.items[meta["row_item"][t]].req_id for t in lr], np.int32)
    embs, emb_req = [], []
    for i, it in enumerate(batch.items):
        if it.kind != EMBED:
            continue
        e = pool_item(pool, it, hf[cu[i]:cu[i + 1]])
        if e is not None:
            embs.append(e)
            emb_req.append(it.req_id)
    emb = np.asarray(embs, dtype).reshape(-1, d)
    return StepOut(logits, logit_req, emb, np.asarray(emb_req, np.int32), x, hf, meta)
