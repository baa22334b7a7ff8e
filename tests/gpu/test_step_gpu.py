"""Whole-step parity through orthrus_step against the oracle: the small
multi-step workload (prefill, then three mixed embedding/decode steps),
LoRA and every pooling head (with and without the L2 flag, and the
buffered head), random ragged batches, the one-layer Mistral-7B-shaped
batch, degenerate batches and host-side error paths."""

import numpy as np
import pytest
import torch

import heterogeneous_embed_decode_amd as hed
from synth import model as sm
from synth import workloads as wl
from tests._gpu import make_pair, run_and_compare, seed_pool

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pool_kind", [wl.POOL_MEAN, wl.POOL_WMEAN, wl.POOL_CLS, wl.POOL_LAST, wl.POOL_BUFFER,
                                       wl.POOL_MEAN | wl.POOL_L2, wl.POOL_LAST | wl.POOL_L2,
                                       wl.POOL_BUFFER | wl.POOL_L2])
def test_tiny_multistep(pool_kind):
    cfg, batches, n_pages = wl.tiny_workload(pool_kind=pool_kind)
    bits = sm.make_weights(cfg, seed=0, gain_std=0.1)
    dev, orc = make_pair(cfg, n_pages, bits, buf_rows=64)
    for s, b in enumerate(batches):
        got, _, _ = run_and_compare(cfg, dev, orc, b, tag=f"tiny pool={pool_kind} step={s}")
        if pool_kind & wl.POOL_L2 and got["emb"].size:
            assert np.allclose(np.linalg.norm(got["emb"].astype(np.float64), axis=1), 1.0, atol=1e-5)
    dev.close()


def test_buffered_head_keeps_rows_and_means_them():
    """BUFFER kind: the slot buffer holds every final hidden state at its
    position (against the oracle), and the emitted vector is the mean of
    exactly those buffered rows (checked against the GPU's own buffer in
    fp64, so the head's arithmetic is checked tightly); a request longer
    than the buffer is refused before any device work.  Two other heads
    (max pooling, attention pooling with a fixed query) run over the GPU's
    buffer agree with the same heads over the oracle's buffer."""
    cfg = sm.TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=6, gain_std=0.1)
    _, batches, n_pages = wl.tiny_workload(cfg=cfg, pool_kind=wl.POOL_BUFFER)
    dev, orc = make_pair(cfg, n_pages, bits, buf_rows=48)
    pool = orc[2]
    from tests._util import rel_l2, cosine
    for s, b in enumerate(batches):
        got, ref, _ = run_and_compare(cfg, dev, orc, b, tag=f"buffer step={s}")
        buf = dev.pool_buf.cpu().numpy()
        for it in b.items:
            if it.kind != wl.EMBED:
                continue
            n = it.ctx_len + it.n_tokens
            assert rel_l2(buf[it.pool_slot, :n], pool["buf"][it.pool_slot, :n]) < 2e-2
        k = 0
        for it in b.items:
            if it.kind == wl.EMBED and it.is_last:
                n = it.ctx_len + it.n_tokens
                mean = buf[it.pool_slot, :n].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(got["emb"][k], mean, rtol=1e-5, atol=1e-6)
                k += 1
                # heads other than the built-in mean, run by the caller over
                # the buffer (the point of keeping every row): max pooling and
                # attention pooling with a fixed query, against the same heads
                # over the oracle's buffered hidden states
                rows_g = buf[it.pool_slot, :n].astype(np.float64)
                rows_o = np.asarray(pool["buf"][it.pool_slot, :n], np.float64)
                qv = np.random.default_rng(it.pool_slot).standard_normal(cfg.d_model)

                def attn_pool(r):
                    a = r @ qv / np.sqrt(cfg.d_model)
                    a = np.exp(a - a.max())
                    return (a / a.sum()) @ r

                for head in (lambda r: r.max(axis=0), attn_pool):
                    hg, ho = head(rows_g), head(rows_o)
                    assert rel_l2(hg, ho) < 2e-2 and cosine(hg, ho) > 0.999
    # a BUFFER item reaching past buf_rows: ECAPACITY, nothing launched
    bb = wl.BatchBuilder(cfg, wl.PageAllocator(n_pages, seed=1))
    bb.add(wl.Request(7, wl.EMBED, list(range(1, 50)), pool_slot=0, pool_kind=wl.POOL_BUFFER))
    big = bb.build([(7, wl.EMBED, 49, 1, 1)])
    before = dev.pool_buf.clone()
    st, _, _ = dev.step(big)
    assert st == hed.ECAPACITY
    torch.cuda.synchronize()
    assert torch.equal(before, dev.pool_buf)
    dev.close()


def test_tiny_lora_mixed_heads():
    cfg = sm.TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=3, gain_std=0.1)
    _, batches, n_pages = wl.tiny_workload(cfg=cfg, pool_kind=wl.POOL_WMEAN, chunk=7)
    dev, orc = make_pair(cfg, n_pages, bits)
    for s, b in enumerate(batches):
        run_and_compare(cfg, dev, orc, b, tag=f"tiny-lora step={s}")
    dev.close()


@pytest.mark.parametrize("scale", [0.5, 2.0])
def test_tiny_lora_scale(scale):
    """Adapter scale other than 1 (folded into the shrink epilogue on the
    GPU): the tiny model's q/k/v sections (64/32/32 columns) share one
    output tile, so the section offsets of the expand K-steps are exercised
    inside a tile; and a d=128 model with rank 16 on a random batch."""
    cfg = sm.TINY.with_(lora_rank=8, lora_scale=scale)
    bits = sm.make_weights(cfg, seed=3, gain_std=0.1)
    _, batches, n_pages = wl.tiny_workload(cfg=cfg, pool_kind=wl.POOL_MEAN, chunk=7)
    dev, orc = make_pair(cfg, n_pages, bits)
    for s, b in enumerate(batches):
        run_and_compare(cfg, dev, orc, b, tag=f"tiny-lora scale={scale} step={s}")
    dev.close()
    base = sm.ModelConfig(n_layers=1, d_model=128, n_q_heads=8, n_kv_heads=2, head_dim=16, ffn_dim=96,
                          vocab=300, lora_rank=16, page_size=8, rope_theta=1e4, lora_scale=scale)
    b, n_pages = wl.random_batch(base, 78, max_items=12, max_len=120, max_ctx=300)
    bits = sm.make_weights(base, seed=8, gain_std=0.1)
    kv = wl.synthetic_kv(base, n_pages, seed=3)
    dev, orc = make_pair(base, n_pages, bits, kv_bits=kv)
    seed_pool(dev, orc, 9)
    run_and_compare(base, dev, orc, b, tag=f"random lora scale={scale}")
    dev.close()


@pytest.mark.parametrize("seed", range(6))
def test_random_ragged_batches(seed):
    base = [sm.TINY.with_(lora_rank=8),
            sm.ModelConfig(n_layers=1, d_model=128, n_q_heads=8, n_kv_heads=1, head_dim=32,
                           ffn_dim=96, vocab=300, lora_rank=16, page_size=5, rope_theta=1e4),
            sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                           ffn_dim=512, vocab=500, lora_rank=8, page_size=16, rope_theta=1e6),
            sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           ffn_dim=384, vocab=1000, lora_rank=16, page_size=16, rope_theta=1e6)][seed % 4]
    kinds = (wl.POOL_MEAN, wl.POOL_WMEAN, wl.POOL_CLS, wl.POOL_LAST, wl.POOL_BUFFER,
             wl.POOL_MEAN | wl.POOL_L2, wl.POOL_BUFFER | wl.POOL_L2, wl.POOL_CLS | wl.POOL_L2)
    b, n_pages = wl.random_batch(base, 100 + seed, max_items=15, max_len=150, max_ctx=700, pool_kinds=kinds)
    bits = sm.make_weights(base, seed=seed, gain_std=0.1)
    kv = wl.synthetic_kv(base, n_pages, seed=3)
    dev, orc = make_pair(base, n_pages, bits, kv_bits=kv, buf_rows=856)
    seed_pool(dev, orc, seed)
    run_and_compare(base, dev, orc, b, tag=f"random seed={seed}")
    dev.close()


def _exact_rows_batch(cfg, seed):
    """512 rows: an embedding chunk that starts its request, a prefill chunk
    after 40 keys and one decode row at context 300 (pages drawn at random)."""
    rng = np.random.default_rng(seed)
    ps = cfg.page_size
    specs = [(wl.EMBED, 300, 0, 1), (wl.PREFILL, 211, 40, 0), (wl.DECODE, 1, 300, 0)]
    n_pages = sum(-(-(n + c) // ps) for _, n, c, _ in specs) + 3
    alloc = wl.PageAllocator(n_pages, seed=seed)
    items, pages = [], []
    for i, (k, n, c, first) in enumerate(specs):
        pg = alloc.alloc(-(-(n + c) // ps))
        items.append(wl.Item(kind=k, req_id=10 + i, n_tokens=n, ctx_len=c, page_off=len(pages), n_pages=len(pg),
                             pool_slot=3 if k == wl.EMBED else -1, pool_kind=wl.POOL_MEAN if k == wl.EMBED else 0,
                             is_first=first, is_last=1))
        pages.extend(pg)
    toks = rng.integers(0, cfg.vocab, 512).astype(np.int32)
    return wl.Batch(items, toks, np.asarray(pages, np.int32)), n_pages


@pytest.mark.parametrize("case", range(5))
def test_qkv_projection_with_rope_epilogue(case):
    """At head dim 128 with an even number of q and KV heads, batches of 512
    rows or more run RoPE and the KV append in the QKV projection's epilogue
    (256-column tiles of two whole heads, rows past the last full tile
    masked).  Ragged row counts, page sizes 5, 16 and 64, the adapter on
    embedding rows and 1, 2 and 4 grouped heads against the oracle, K/V
    pages included; case 4 is 511 rows, which takes the separate RoPE
    kernel, beside case 3 at exactly 512."""
    cfgs = [sm.ModelConfig(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=128, ffn_dim=384,
                           vocab=1000, lora_rank=8, page_size=5, rope_theta=1e6),
            sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=384,
                           vocab=1000, lora_rank=16, page_size=16, rope_theta=1e4),
            sm.ModelConfig(n_layers=1, d_model=384, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn_dim=256,
                           vocab=700, lora_rank=0, page_size=64, rope_theta=1e6)]
    if case < 3:
        cfg = cfgs[case]
        b, n_pages = wl.random_batch(cfg, (209, 208, 218)[case], max_items=15, max_len=220, max_ctx=500)
    else:
        cfg = cfgs[0]
        b, n_pages = _exact_rows_batch(cfg, 7)
        if case == 4:
            it = b.items[1]
            b.items[1] = wl.Item(kind=it.kind, req_id=it.req_id, n_tokens=it.n_tokens - 1, ctx_len=it.ctx_len,
                                 page_off=it.page_off, n_pages=it.n_pages, is_last=1)
            b = wl.Batch(b.items, np.delete(b.token_ids, 400), b.page_ids)
    print(f"qkv+rope case {case}: rows={b.n_tokens} hd={cfg.head_dim} Hq={cfg.n_q_heads} "
          f"Hkv={cfg.n_kv_heads} ps={cfg.page_size}", flush=True)
    assert (b.n_tokens >= 512) == (case != 4)
    bits = sm.make_weights(cfg, seed=case, gain_std=0.1)
    kv = wl.synthetic_kv(cfg, n_pages, seed=3)
    dev, orc = make_pair(cfg, n_pages, bits, kv_bits=kv, max_tokens=2048)
    seed_pool(dev, orc, case)
    run_and_compare(cfg, dev, orc, b, tag=f"qkv+rope case={case}")
    dev.close()


@pytest.mark.parametrize("pool_kind", [wl.POOL_LAST, wl.POOL_BUFFER | wl.POOL_L2])
def test_one_mistral_layer_full_batch(pool_kind):
    # the one-layer batch as bench.py runs it (default last-token pooling, and
    # --pool-kind buffer+l2)
    cfg, batch, n_pages = wl.one_layer_workload(pool_kind=pool_kind)
    print(f"one-layer: rows={batch.n_tokens} pages={n_pages} pool={pool_kind}", flush=True)
    bits = sm.make_weights(cfg, seed=0)
    kv = wl.synthetic_kv(cfg, n_pages, seed=3)
    buf = 512 if (pool_kind & ~wl.POOL_L2) == wl.POOL_BUFFER else 0
    dev, orc = make_pair(cfg, n_pages, bits, kv_bits=kv, max_tokens=8192, max_items=128, buf_rows=buf)
    got, _, _ = run_and_compare(cfg, dev, orc, batch, tag="one-layer")
    if pool_kind & wl.POOL_L2:
        assert np.allclose(np.linalg.norm(got["emb"].astype(np.float64), axis=1), 1.0, atol=1e-5)
    dev.close()


def test_degenerate_batches_and_errors():
    cfg = sm.TINY.with_(lora_rank=8)
    bits = sm.make_weights(cfg, seed=1, gain_std=0.1)
    n_pages = 40
    dev, orc = make_pair(cfg, n_pages, bits)
    # empty batch: nothing to do, OK
    empty = wl.Batch([], np.zeros(0, np.int32), np.zeros(0, np.int32))
    st, nl, ne = dev.step(empty)
    assert (st, nl, ne) == (hed.OK, 0, 0)
    # decode at context 0, a one-token embedding chunk, a one-token prefill
    alloc = wl.PageAllocator(n_pages, seed=2)
    bb = wl.BatchBuilder(cfg, alloc)
    bb.add(wl.Request(1, wl.EMBED, [5], pool_slot=0, pool_kind=wl.POOL_CLS))
    bb.add(wl.Request(2, wl.PREFILL, [7, 8]))
    bb.add(wl.Request(3, wl.DECODE, [9]))
    b = bb.build([(1, wl.EMBED, 1, 1, 1), (2, wl.PREFILL, 1, 1, 1), (3, wl.DECODE, 1, 0, 1)])
    run_and_compare(cfg, dev, orc, b, tag="degenerate")
    # invalid batch: error before any device work, KV untouched
    before = dev.K.clone()
    bad = wl.Batch([wl.Item(kind=wl.DECODE, req_id=1, n_tokens=1, ctx_len=0, page_off=0, n_pages=1),
                    wl.Item(kind=wl.EMBED, req_id=2, n_tokens=1, ctx_len=0, page_off=1, n_pages=1,
                            pool_slot=0, is_first=1, is_last=1)],
                   np.array([1, 2], np.int32), np.array([3, 4], np.int32))
    st, _, _ = dev.step(bad)
    assert st == hed.EINVAL
    assert "sorted" in hed.orthrus_last_error(dev.eng)
    torch.cuda.synchronize()
    assert torch.equal(before, dev.K)
    # output capacity
    small = wl.Batch([wl.Item(kind=wl.DECODE, req_id=i, n_tokens=1, ctx_len=0, page_off=i, n_pages=1)
                      for i in range(3)], np.array([1, 2, 3], np.int32), np.array([0, 1, 2], np.int32))
    a = dev.step_args(small)
    st, _, _ = hed.orthrus_step(dev.eng, a, dev.pool_sum.data_ptr(), dev.pool_wsum.data_ptr(),
                                dev.pool_kept.data_ptr(), dev.logits.data_ptr(), 2, dev.emb.data_ptr(),
                                4, None, None)
    assert st == hed.ECAPACITY
    dev.close()


@pytest.mark.parametrize("seed,tid,start,n", [(3, 0, 0, 100003), (3, 1, 123456789012, 4097), (7, 2, 2**33 + 5, 70000)])
def test_hash_fill_matches_numpy_definition(seed, tid, start, n):
    from synth.hashfill import splitmix64_fill
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    assert hed.orthrus_fill_hash_bf16(out.data_ptr(), n, seed, tid, start,
                                      torch.cuda.current_stream().cuda_stream) == hed.OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), splitmix64_fill(seed, tid, n, start))
