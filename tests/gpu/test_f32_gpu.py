"""The fp32 path (model dtype "f32": fp32 weights, KV pages, activations and
accumulation) against the oracle in fp64, every output row to rel-L2 1e-5:
the tiny fp32 decoder of the small correctness workload (prefill, then three
mixed embedding/decode steps) under every pooling head, and random ragged
fp32 batches with prior KV, mid-request pooling state, the LoRA adapter at
scales other than 1, every head dim and GQA group size."""

import numpy as np
import pytest

import oracle
from synth import model as sm
from synth import workloads as wl
from synth.bf16 import bf16_bits_to_f32
from tests._gpu import make_pair, seed_pool
from tests._util import row_rel_l2, cosine

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


def _compare(cfg, dev, orc, batch, tag):
    W, kv, pool = orc
    print(f"[f32 {tag}] items={batch.n_items} rows={batch.n_tokens}", flush=True)
    got = dev.step_checked(batch, want_hidden=True)
    ref = oracle.step(cfg, W, batch, kv, pool, np.float64)
    assert np.array_equal(got["logit_req"], ref.logit_req) and np.array_equal(got["emb_req"], ref.emb_req)
    res = {"hidden_row_max": float(row_rel_l2(got["hidden"], ref.hidden).max())}
    if ref.logits.size:
        res["logit_row_max"] = float(row_rel_l2(got["logits"], ref.logits).max())
    if ref.emb.size:
        res["emb_row_max"] = float(row_rel_l2(got["emb"], ref.emb).max())
        res["emb_cos_min"] = min(cosine(got["emb"][i], ref.emb[i]) for i in range(ref.emb.shape[0]))
    slots, ps = ref.meta["slot"], cfg.page_size
    kv_max = 0.0
    for l in range(cfg.n_layers):
        for tens, okv in ((dev.K, kv[0]), (dev.V, kv[1])):
            g = tens[l].cpu().numpy()[slots // ps, :, slots % ps, :]
            kv_max = max(kv_max, float(row_rel_l2(g, okv[l][slots // ps, :, slots % ps, :]).max()))
    res["kv_row_max"] = kv_max
    print(f"[f32 {tag}] {res}", flush=True)
    for k in ("hidden_row_max", "logit_row_max", "emb_row_max", "kv_row_max"):
        assert res.get(k, 0.0) < F32_TOL, (tag, res)
    assert res.get("emb_cos_min", 1.0) > 1 - 1e-9, (tag, res)
    return got


@pytest.mark.parametrize("pool_kind", [wl.POOL_MEAN, wl.POOL_WMEAN, wl.POOL_CLS, wl.POOL_LAST,
                                       wl.POOL_BUFFER | wl.POOL_L2])
def test_tiny_fp32_decoder(pool_kind):
    cfg, batches, n_pages = wl.tiny_workload(cfg=sm.TINY_F32, pool_kind=pool_kind)
    bits = sm.make_weights(cfg, seed=0)
    assert all(v.dtype == np.float32 for v in bits.values())
    dev, orc = make_pair(cfg, n_pages, bits, oracle_dtype=np.float64, buf_rows=64)
    for s, b in enumerate(batches):
        _compare(cfg, dev, orc, b, f"tiny pool={pool_kind} step={s}")
    dev.close()


BASES = [
    sm.TINY_F32.with_(lora_rank=8, lora_scale=2.0),
    sm.ModelConfig(n_layers=1, d_model=128, n_q_heads=8, n_kv_heads=1, head_dim=32, ffn_dim=96, vocab=300,
                   lora_rank=16, page_size=5, rope_theta=1e4, lora_scale=0.5, dtype="f32"),
    sm.ModelConfig(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=200, vocab=500,
                   lora_rank=8, page_size=16, rope_theta=1e6, dtype="f32"),
    sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=384, vocab=1000,
                   lora_rank=16, page_size=16, rope_theta=1e6, dtype="f32"),
]


@pytest.mark.parametrize("seed", range(4))
def test_fp32_random_ragged(seed):
    base = BASES[seed]
    kinds = (wl.POOL_MEAN, wl.POOL_WMEAN, wl.POOL_CLS, wl.POOL_LAST, wl.POOL_BUFFER, wl.POOL_MEAN | wl.POOL_L2)
    b, n_pages = wl.random_batch(base, 200 + seed, max_items=15, max_len=120, max_ctx=600, pool_kinds=kinds)
    bits = sm.make_weights(base, seed=seed, gain_std=0.1)
    kv = wl.synthetic_kv(base, n_pages, seed=3)
    dev, orc = make_pair(base, n_pages, bits, kv_bits=kv, oracle_dtype=np.float64, buf_rows=800)
    assert dev.K.dtype.is_floating_point and dev.K.element_size() == 4
    # prior KV as fp32 values: the same numbers on both sides
    assert np.array_equal(dev.K[0].cpu().numpy(), bf16_bits_to_f32(kv[0][0]))
    seed_pool(dev, orc, seed)
    _compare(base, dev, orc, b, f"random seed={seed}")
    dev.close()
