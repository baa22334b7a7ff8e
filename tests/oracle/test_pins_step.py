"""Pins of the oracle's whole step against what the pages and the maths fix:
chunked pooling equals a single pass (Table 7 bar), a decode row equals
full recomputation, CLS equals a one-token forward, the LoRA adapter
touches embedding rows only, requests are independent of their batch
neighbours and of page placement, and degenerate weights reduce the model
to closed forms."""

import json
import os

import numpy as np
import pytest

import oracle
from synth import model as sm
from synth import workloads as wl
from synth.workloads import Item, Batch, PageAllocator, BatchBuilder, Request
from tests._util import OracleRunner, MINI, rel_l2, cosine, single_request_batches

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "..", "golden",
                                   "pooling_equivalence.json")))
TINY = sm.TINY


def _embed(cfg, tokens, chunk, kind, dtype, bits):
    batches, n_pages = single_request_batches(cfg, tokens, chunk, pool_kind=kind)
    run = OracleRunner(cfg, n_pages, dtype=dtype, weights=bits)
    out = None
    for b in batches:
        out = run.step(b)
    assert out.emb.shape[0] == 1
    return out.emb[0]


@pytest.mark.parametrize("kind", [wl.POOL_MEAN, wl.POOL_WMEAN, wl.POOL_CLS, wl.POOL_LAST])
def test_chunked_equals_single_pass_fp64_tiny(kind):
    bits = sm.make_weights(TINY.with_(lora_rank=8), seed=0, gain_std=0.1)
    cfg = TINY.with_(lora_rank=8)
    toks = np.random.default_rng(11).integers(0, cfg.vocab, 40)
    one = _embed(cfg, toks, 40, kind, np.float64, bits)
    for C in (16, 7, 1):
        ch = _embed(cfg, toks, C, kind, np.float64, bits)
        assert rel_l2(ch, one) < 1e-12, (kind, C)


def test_chunked_equals_single_pass_table7_bar_fp32():
    """Stand-in for the page's 250-sample study (samples unpublished):
    seeded inputs of 300-1500 tokens on a 4-layer d=128 model, fp32."""
    bits = sm.make_weights(MINI, seed=0, gain_std=0.1)
    rng = np.random.default_rng(2)
    lengths = [300, 700, 1100, 1500]
    heads = {"mean": wl.POOL_MEAN, "cls": wl.POOL_CLS, "wmean": wl.POOL_WMEAN}
    errs, coss = [], []
    for n in lengths:
        toks = rng.integers(0, MINI.vocab, n)
        for name in GOLD["heads"]:
            k = heads[name]
            one = _embed(MINI, toks, n, k, np.float32, bits)
            for C in GOLD["chunk_sizes"]:
                if C >= n:
                    continue
                ch = _embed(MINI, toks, C, k, np.float32, bits)
                errs.append(rel_l2(ch, one))
                coss.append(cosine(ch, one))
    assert min(coss) > GOLD["min_cosine_exceeds"]
    assert np.mean(errs) < GOLD["mean_rel_l2_below"]
    assert np.percentile(errs, 99) < GOLD["p99_rel_l2_below"]


def _prefill_then_decode(cfg, bits, toks, c, dtype=np.float64):
    """Prefill c tokens, then decode token c; return decode logits and
    the logits of one prefill over all c+1 tokens (last row)."""
    alloc = PageAllocator(32, seed=4)
    bb = BatchBuilder(cfg, alloc)
    bb.add(Request(1, wl.PREFILL, list(toks)))
    run = OracleRunner(cfg, 32, dtype=dtype, weights=bits)
    b = bb.build([(1, wl.PREFILL, c, 1, 1)])
    run.step(b)
    bb.commit(b)
    b = bb.build([(1, wl.DECODE, 1, 0, 1)])
    dec = run.step(b).logits[0]
    alloc2 = PageAllocator(32, seed=9)
    bb2 = BatchBuilder(cfg, alloc2)
    bb2.add(Request(1, wl.PREFILL, list(toks)))
    run2 = OracleRunner(cfg, 32, dtype=dtype, weights=bits)
    full = run2.step(bb2.build([(1, wl.PREFILL, c + 1, 1, 1)])).logits[0]
    return dec, full


@pytest.mark.parametrize("c", [30, 50])
def test_decode_equals_recompute(c):
    bits = sm.make_weights(TINY, seed=0, gain_std=0.1)
    toks = np.random.default_rng(c).integers(0, TINY.vocab, c + 1)
    dec, full = _prefill_then_decode(TINY, bits, toks, c)
    assert rel_l2(dec, full) < 1e-12


def test_cls_equals_one_token_forward():
    cfg = TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=0, gain_std=0.1)
    toks = np.random.default_rng(5).integers(0, cfg.vocab, 33)
    cls = _embed(cfg, toks, 16, wl.POOL_CLS, np.float64, bits)
    one = _embed(cfg, toks[:1], 1, wl.POOL_LAST, np.float64, bits)
    assert rel_l2(cls, one) < 1e-13


def _mixed_batch(cfg, seed_pages=4, n_pages=64, order=None):
    """Two embedding chunks, one prefill chunk, two decode rows."""
    rng = np.random.default_rng(21)
    alloc = PageAllocator(n_pages, seed=seed_pages)
    bb = BatchBuilder(cfg, alloc)
    bb.add(Request(0, wl.EMBED, list(rng.integers(0, cfg.vocab, 20)), pool_slot=0))
    bb.add(Request(1, wl.EMBED, list(rng.integers(0, cfg.vocab, 11)), pool_slot=1,
                   pool_kind=wl.POOL_WMEAN))
    bb.add(Request(2, wl.PREFILL, list(rng.integers(0, cfg.vocab, 13))))
    bb.add(Request(3, wl.PREFILL, list(rng.integers(0, cfg.vocab, 9))))
    bb.add(Request(4, wl.PREFILL, list(rng.integers(0, cfg.vocab, 6))))
    # give the decode requests some context via a first step
    pre = bb.build([(3, wl.PREFILL, 8, 1, 1), (4, wl.PREFILL, 5, 1, 1)])
    bb.commit(pre)
    entries = [(0, wl.EMBED, 20, 1, 1), (1, wl.EMBED, 11, 1, 1), (2, wl.PREFILL, 13, 1, 1),
               (3, wl.DECODE, 1, 0, 1), (4, wl.DECODE, 1, 0, 1)]
    if order is not None:
        entries = [entries[i] for i in order]
    return pre, bb.build(entries)


def _run_pair(cfg, bits, pre, b, n_pages=64):
    run = OracleRunner(cfg, n_pages, dtype=np.float64, weights=bits)
    run.step(pre)
    return run.step(b)


def test_lora_zero_b_is_base_and_generation_rows_ignore_adapter():
    cfg = TINY.with_(lora_rank=8)
    with_ad = sm.make_weights(cfg, seed=0, gain_std=0.1)
    zero_b = sm.make_weights(cfg, seed=0, gain_std=0.1, zero_lora_b=True)
    base = dict(zero_b)
    for k in base:
        if ".lora_a" in k:
            base[k] = np.zeros_like(base[k])
    pre, b = _mixed_batch(cfg)
    o_ad = _run_pair(cfg, with_ad, pre, b)
    o_zb = _run_pair(cfg, zero_b, pre, b)
    o_base = _run_pair(cfg, base, pre, b)
    # zero expand matrix: identical to the base model everywhere
    np.testing.assert_array_equal(o_zb.logits, o_base.logits)
    np.testing.assert_array_equal(o_zb.emb, o_base.emb)
    # the adapter changes embedding outputs ...
    assert rel_l2(o_ad.emb, o_base.emb) > 1e-3
    # ... and leaves generation rows bit-identical
    np.testing.assert_array_equal(o_ad.logits, o_base.logits)


def test_requests_are_independent_of_batch_and_pages():
    cfg = TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=0, gain_std=0.1)
    pre, b = _mixed_batch(cfg)
    full = _run_pair(cfg, bits, pre, b)
    pre2, b2 = _mixed_batch(cfg, seed_pages=99, n_pages=80)
    moved = _run_pair(cfg, bits, pre2, b2, n_pages=80)
    np.testing.assert_allclose(moved.logits, full.logits, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(moved.emb, full.emb, rtol=1e-12, atol=1e-12)
    # each item alone in its batch gives the same outputs
    for i, it in enumerate(b.items):
        sub = Batch([Item(**{**it.__dict__, "page_off": 0})],
                    b.token_ids[sum(x.n_tokens for x in b.items[:i]):][:it.n_tokens],
                    b.item_pages(i))
        run = OracleRunner(cfg, 64, dtype=np.float64, weights=bits)
        run.step(pre)
        o = run.step(sub)
        if it.kind == wl.EMBED:
            j = [x.req_id for x in b.items if x.kind == wl.EMBED].index(it.req_id)
            np.testing.assert_allclose(o.emb[0], full.emb[j], rtol=1e-12, atol=1e-12)
        else:
            j = list(full.logit_req).index(it.req_id)
            np.testing.assert_allclose(o.logits[0], full.logits[j], rtol=1e-12, atol=1e-12)


def test_future_tokens_do_not_change_earlier_rows():
    bits = sm.make_weights(TINY, seed=0, gain_std=0.1)
    toks = np.random.default_rng(3).integers(0, TINY.vocab, 24)
    toks2 = toks.copy()
    toks2[20:] = (toks2[20:] + 17) % TINY.vocab
    outs = []
    for t in (toks, toks2):
        bs, npg = single_request_batches(TINY, t, 24, kind=wl.PREFILL)
        outs.append(OracleRunner(TINY, npg, weights=bits).step(bs[0]).final)
    np.testing.assert_array_equal(outs[0][:20], outs[1][:20])
    assert not np.allclose(outs[0][20:], outs[1][20:])


def test_zero_blocks_reduce_to_norm_and_lm_head():
    """With W_o = W_down = 0 every layer is the identity on the residual
    stream, so the final state is the token embedding itself."""
    bits = sm.make_weights(TINY, seed=0, gain_std=0.1)
    for l in range(TINY.n_layers):
        bits[f"layers.{l}.w_o"][:] = 0
        bits[f"layers.{l}.w_down"][:] = 0
    toks = np.random.default_rng(4).integers(0, TINY.vocab, 10)
    bs, npg = single_request_batches(TINY, toks, 10, kind=wl.PREFILL)
    run = OracleRunner(TINY, npg, weights=bits)
    out = run.step(bs[0])
    E = run.W["tok_emb"][toks]
    np.testing.assert_array_equal(out.hidden, E)
    g = run.W["g_final"]
    hf = E / np.sqrt((E * E).mean(-1, keepdims=True) + TINY.rms_eps) * g
    np.testing.assert_allclose(out.logits[0], run.W["lm_head"] @ hf[-1], rtol=1e-12)


def test_single_token_layer_is_value_path():
    """One token: attention returns that token's value (kv head h // group),
    so the attention block adds rope-free v_{h//grp} W_o^T to the residual."""
    cfg = TINY.with_(n_layers=1)
    bits = sm.make_weights(cfg, seed=0, gain_std=0.1)
    bits["layers.0.w_down"][:] = 0
    bs, npg = single_request_batches(cfg, [17], 1, kind=wl.PREFILL)
    run = OracleRunner(cfg, npg, weights=bits)
    out = run.step(bs[0])
    W = run.W
    x0 = W["tok_emb"][17]
    h = x0 / np.sqrt((x0 * x0).mean() + cfg.rms_eps) * W["layers.0.g_attn"]
    v = (W["layers.0.w_qkv"][cfg.q_dim + cfg.kv_dim:] @ h).reshape(cfg.n_kv_heads, cfg.head_dim)
    grp = cfg.n_q_heads // cfg.n_kv_heads
    o = np.concatenate([v[hq // grp] for hq in range(cfg.n_q_heads)])
    expect = x0 + W["layers.0.w_o"] @ o
    np.testing.assert_allclose(out.hidden[0], expect, rtol=1e-12, atol=1e-14)


def test_kv_written_for_every_row_at_its_slot():
    cfg = TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=0, gain_std=0.1)
    pre, b = _mixed_batch(cfg)
    run = OracleRunner(cfg, 64, dtype=np.float64, weights=bits)
    run.step(pre)
    out = run.step(b)
    slots = out.meta["slot"]
    ps = cfg.page_size
    for l in range(cfg.n_layers):
        written = run.kv[0][l][slots // ps, :, slots % ps, :]
        assert np.all(np.abs(written).sum(axis=(1, 2)) > 0)
