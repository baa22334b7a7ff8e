"""Closed-form pins of the oracle's LoRA delta and feed-forward block.

The adapter of the embedding model (full text §2.2 Parameter sharing, §5.1:
the embedding requests run the shared backbone plus a LoRA adapter) and the
SwiGLU feed-forward of the shared forward (§3.1) are pinned with one-hot
weights: each adapter section (q, k, v, o) and each feed-forward factor
(gate, up, down) moves exactly one coordinate, chosen distinct, so a
section mix-up, a dropped or doubled scale, a gate/up swap, the wrong norm
gain or the wrong block input lands on a different coordinate or value.

With the q and k projections at zero every attention score is zero, so a
row at position p attends uniformly to positions 0..p and its attention
output is the running mean of the values (a softmax special case).
"""

import numpy as np
import pytest

import oracle
from synth import model as sm
from synth import workloads as wl
from synth.bf16 import f32_to_bf16_bits
from synth.workloads import PageAllocator, BatchBuilder, Request

CFG = sm.TINY.with_(n_layers=1, lora_rank=8)     # d 64, qd 64, kvd 32, F 176
QD, KD, R = CFG.q_dim, CFG.kv_dim, CFG.lora_rank
GRP = CFG.n_q_heads // CFG.n_kv_heads


def _bits(v):
    return f32_to_bf16_bits(np.array([v], np.float32))[0]


def _weights(seed=4):
    """Random gains (so g_attn and g_ffn differ), every matrix zero."""
    w = sm.make_weights(CFG, seed=seed, gain_std=0.1)
    for k in w:
        if not k.split(".")[-1].startswith("g_") and k.startswith("layers."):
            w[k][:] = 0
    return w


def _batch():
    """Two embedding chunks (4 and 3 tokens, context 0), one 5-token prefill
    chunk and one decode row at context 0: embedding rows are 0..6."""
    rng = np.random.default_rng(8)
    bb = BatchBuilder(CFG, PageAllocator(16, seed=3))
    bb.add(Request(0, wl.EMBED, list(rng.integers(0, CFG.vocab, 4)), pool_slot=0))
    bb.add(Request(1, wl.EMBED, list(rng.integers(0, CFG.vocab, 3)), pool_slot=1))
    bb.add(Request(2, wl.PREFILL, list(rng.integers(0, CFG.vocab, 5))))
    bb.add(Request(3, wl.DECODE, list(rng.integers(0, CFG.vocab, 1))))
    return bb.build([(0, wl.EMBED, 4, 1, 1), (1, wl.EMBED, 3, 1, 1), (2, wl.PREFILL, 5, 1, 1),
                     (3, wl.DECODE, 1, 0, 1)])


def _run(cfg, bits, batch):
    W = oracle.widen_weights(bits, np.float64)
    kv = oracle.new_kv(cfg, 16, np.float64)
    pool = oracle.new_pool(4, cfg.d_model, np.float64)
    trace = []
    out = oracle.step(cfg, W, batch, kv, pool, np.float64, trace=trace)
    out.kv = kv
    return W, out, trace[0]


def _item_rows(batch):
    """(first row, n rows) of every item, in row order."""
    rows, t = [], 0
    for it in batch.items:
        rows.append((t, it.n_tokens))
        t += it.n_tokens
    return rows


def _running_mean(col, batch):
    """Per row, the mean of col over its item's rows up to and including it
    (every item here starts at context 0)."""
    out = np.zeros_like(col)
    for r0, n in _item_rows(batch):
        out[r0:r0 + n] = np.cumsum(col[r0:r0 + n]) / np.arange(1, n + 1)
    return out


@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_lora_qkv_sections_one_hot(scale):
    """A_q/A_k/A_v pick input features f_q/f_k/f_v into adapter ranks
    j_q/j_k/j_v; B puts rank j_sec on output column c_sec of its own
    section.  Embedding rows get s * h[f_sec] at c_sec and nothing else;
    generation rows get nothing."""
    cfg = CFG.with_(lora_scale=scale)
    bits = _weights()
    f = {"q": 3, "k": 17, "v": 40}
    j = {"q": 1, "k": 6, "v": 3}
    c = {"q": 9, "k": QD + 21, "v": QD + KD + 5}
    for n, sec in (("q", 0), ("k", 1), ("v", 2)):
        bits["layers.0.lora_a_qkv"][sec * R + j[n], f[n]] = _bits(1.0)
        bits["layers.0.lora_b_qkv"][c[n], j[n]] = _bits(1.0)
    b = _batch()
    W, out, tr = _run(cfg, bits, b)
    TE = out.meta["n_embed_rows"]
    assert TE == 7
    x0 = W["tok_emb"][b.token_ids]
    h = oracle.rmsnorm(x0, W["layers.0.g_attn"], cfg.rms_eps)
    expect = np.zeros((b.n_tokens, cfg.qkv_dim))
    for n in ("q", "k", "v"):
        expect[:TE, c[n]] = scale * h[:TE, f[n]]
    np.testing.assert_allclose(tr["qkv"], expect, rtol=1e-13, atol=1e-15)
    # k at position 0 (RoPE is the identity there) and v reach the cache
    hd = cfg.head_dim
    p0 = b.item_pages(0)[0]
    K0, V0 = out.kv[0][0], out.kv[1][0]
    kc, vc = c["k"] - QD, c["v"] - QD - KD
    assert K0[p0, kc // hd, 0, kc % hd] == scale * h[0, f["k"]]
    assert V0[p0, vc // hd, 0, vc % hd] == scale * h[0, f["v"]]
    assert np.count_nonzero(V0) == 7 and np.count_nonzero(K0[p0, :, 0, :]) == 1


@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_lora_o_one_hot_and_uniform_attention(scale):
    """v = h[f_v] on one value column; q = k = 0 make attention the running
    mean of v; the output adapter maps attention column a (a query head
    reading that value column through the GQA map) to residual column c
    through rank j with scale s.  W_o = W_down = 0, so the final residual
    is the token embedding plus s * mean_{p<=t} h[p, f_v] at column c, on
    embedding rows only."""
    cfg = CFG.with_(lora_scale=scale)
    bits = _weights()
    hd = cfg.head_dim
    f_v, vcol = 11, 1 * hd + 7                   # kv head 1, dim 7
    a = (1 * GRP + 1) * hd + 7                   # query head 3 reads kv head 1
    jr, c = 5, 30
    bits["layers.0.w_qkv"][QD + KD + vcol, f_v] = _bits(1.0)
    bits["layers.0.lora_a_o"][jr, a] = _bits(1.0)
    bits["layers.0.lora_b_o"][c, jr] = _bits(1.0)
    b = _batch()
    W, out, tr = _run(cfg, bits, b)
    TE = out.meta["n_embed_rows"]
    x0 = W["tok_emb"][b.token_ids]
    h = oracle.rmsnorm(x0, W["layers.0.g_attn"], cfg.rms_eps)
    m = _running_mean(h[:, f_v], b)
    # attention output: every query head of kv group 1 carries the running mean
    o = tr["o"].reshape(b.n_tokens, cfg.n_q_heads, hd)
    for hq in range(cfg.n_q_heads):
        want = m if hq // GRP == 1 else np.zeros_like(m)
        np.testing.assert_allclose(o[:, hq, 7], want, rtol=1e-13, atol=1e-15)
    expect = x0.copy()
    expect[:TE, c] += scale * m[:TE]
    np.testing.assert_allclose(out.hidden, expect, rtol=1e-13, atol=1e-15)


def test_lora_scale_is_linear():
    """Doubling the scale doubles the adapter's change of every embedding
    output of a random adapter; generation rows never change."""
    outs = {}
    bits = sm.make_weights(CFG, seed=2, gain_std=0.1)
    base_bits = dict(bits)
    base_bits["layers.0.lora_b_qkv"] = np.zeros_like(bits["layers.0.lora_b_qkv"])
    base_bits["layers.0.lora_b_o"] = np.zeros_like(bits["layers.0.lora_b_o"])
    b = _batch()
    for s in (0.5, 1.0):
        _, out, tr = _run(CFG.with_(lora_scale=s), bits, b)
        outs[s] = tr["qkv"]
    _, out0, tr0 = _run(CFG, base_bits, b)
    d_half = outs[0.5] - tr0["qkv"]
    d_one = outs[1.0] - tr0["qkv"]
    TE = out0.meta["n_embed_rows"]
    np.testing.assert_allclose(d_one[:TE], 2 * d_half[:TE], rtol=1e-10, atol=1e-14)
    assert np.abs(d_one[:TE]).max() > 1e-3
    np.testing.assert_array_equal(d_one[TE:], 0)


@pytest.mark.parametrize("attn_col", [None, 25])
def test_ffn_one_hot_swiglu(attn_col):
    """Gate row i reads feature fa with weight alpha, up row i reads fb with
    weight beta, the down projection writes unit i to residual column c2:
    the block adds silu(alpha h2[fa]) * beta h2[fb] at c2, where h2 is the
    FFN norm (gain g_ffn) of the residual after attention.  With attn_col
    set, the attention block first adds the running mean of h[f_v] at that
    column (W_o one-hot), so the FFN input differs from the embedding."""
    cfg = CFG.with_(lora_rank=0)
    bits = sm.make_weights(cfg, seed=4, gain_std=0.1)
    for k in bits:
        if k.startswith("layers.") and not k.split(".")[-1].startswith("g_"):
            bits[k][:] = 0
    F, hd = cfg.ffn_dim, cfg.head_dim
    alpha, beta = 1.5, -0.625
    i_unit, fa, fb, c2 = 101, 25, 48, 7
    f_v, vcol = 11, 0 * hd + 3
    a = 1 * hd + 3                                 # query head 1 reads kv head 0
    if attn_col is not None:
        bits["layers.0.w_qkv"][QD + KD + vcol, f_v] = _bits(1.0)
        bits["layers.0.w_o"][attn_col, a] = _bits(1.0)
    bits["layers.0.w_gate_up"][i_unit, fa] = _bits(alpha)
    bits["layers.0.w_gate_up"][F + i_unit, fb] = _bits(beta)
    bits["layers.0.w_down"][c2, i_unit] = _bits(1.0)
    b = _batch()
    W, out, tr = _run(cfg, bits, b)
    x0 = W["tok_emb"][b.token_ids]
    x_attn = x0.copy()
    if attn_col is not None:
        h = oracle.rmsnorm(x0, W["layers.0.g_attn"], cfg.rms_eps)
        x_attn[:, attn_col] += _running_mean(h[:, f_v], b)
    np.testing.assert_allclose(tr["x_attn"], x_attn, rtol=1e-13, atol=1e-15)
    g = W["layers.0.g_ffn"]
    assert not np.allclose(g, W["layers.0.g_attn"])
    h2 = x_attn / np.sqrt((x_attn * x_attn).mean(-1, keepdims=True) + cfg.rms_eps) * g
    gate, up = alpha * h2[:, fa], beta * h2[:, fb]
    unit = gate / (1.0 + np.exp(-gate)) * up
    expect = x_attn.copy()
    expect[:, c2] += unit
    np.testing.assert_allclose(tr["act"][:, i_unit], unit, rtol=1e-13, atol=1e-15)
    assert np.count_nonzero(tr["act"]) == np.count_nonzero(unit)
    np.testing.assert_allclose(out.hidden, expect, rtol=1e-13, atol=1e-15)
    # the swapped reading (silu on the up factor) would differ here
    swapped = up / (1.0 + np.exp(-up)) * gate
    assert np.abs(swapped - unit).max() > 1e-2
