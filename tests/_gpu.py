"""GPU test helpers: run the same seeded workload through the library and
through the oracle, and compare."""

import numpy as np

import oracle
from synth import model as sm
from synth import workloads as wl
from tests._util import rel_l2, cosine

# Acceptance bars: rel-L2 on logits and hidden states, cosine on pooled
# embeddings (bf16 compute against the fp32 oracle).
LOGIT_TOL = 2e-2
HIDDEN_TOL = 2e-2
EMB_COS = 0.999


def make_pair(dims, n_pages, weights, kv_bits=None, max_tokens=None, max_items=64, slots=16,
              oracle_dtype=np.float32):
    from heterogeneous_embed_decode_amd.device_model import DeviceModel
    mt = max_tokens or 4096
    dev = DeviceModel(dims, weights, n_pages, mt, max_items, slots, kv_bits=kv_bits)
    W = oracle.widen_weights(weights, oracle_dtype)
    if kv_bits is None:
        kv = oracle.new_kv(dims, n_pages, oracle_dtype)
    else:
        kv = oracle.new_kv(dims, n_pages, oracle_dtype, kv_bits[0], kv_bits[1])
    pool = oracle.new_pool(slots, dims.d_model, oracle_dtype)
    return dev, (W, kv, pool)


def seed_pool(dev, orc, seed=5):
    """Same synthetic prior pooling state on both sides (mid-request chunks)."""
    import torch
    W, kv, pool = orc
    rng = np.random.default_rng(seed)
    S, d = pool["sum"].shape
    sm_ = rng.standard_normal((S, d)).astype(np.float32) * 10
    ws = rng.integers(1, 500, S).astype(np.float32)
    kp = rng.standard_normal((S, d)).astype(np.float32)
    pool["sum"][:] = sm_
    pool["wsum"][:] = ws
    pool["kept"][:] = kp
    dev.pool_sum[:S].copy_(torch.from_numpy(sm_))
    dev.pool_wsum[:S].copy_(torch.from_numpy(ws))
    dev.pool_kept[:S].copy_(torch.from_numpy(kp))


def run_and_compare(dims, dev, orc, batch, check_kv=True, dtype=np.float32, tag=""):
    W, kv, pool = orc
    print(f"[step {tag}] items={batch.n_items} rows={batch.n_tokens}", flush=True)
    got = dev.step_checked(batch, want_hidden=True)
    ref = oracle.step(dims, W, batch, kv, pool, dtype)
    res = {}
    assert got["logits"].shape == ref.logits.shape, (got["logits"].shape, ref.logits.shape)
    assert got["emb"].shape == ref.emb.shape, (got["emb"].shape, ref.emb.shape)
    res["hidden"] = rel_l2(got["hidden"], ref.hidden)
    if ref.logits.size:
        res["logits"] = rel_l2(got["logits"], ref.logits)
        for i in range(ref.logits.shape[0]):
            assert rel_l2(got["logits"][i], ref.logits[i]) < LOGIT_TOL, (tag, "logit row", i)
    if ref.emb.size:
        res["emb_cos_min"] = min(cosine(got["emb"][i], ref.emb[i]) for i in range(ref.emb.shape[0]))
        assert res["emb_cos_min"] >= EMB_COS, (tag, res)
    assert res["hidden"] < HIDDEN_TOL, (tag, res)
    if check_kv:
        from synth.bf16 import bf16_bits_to_f32
        slots = ref.meta["slot"]
        ps = dims.page_size
        for l in range(dims.n_layers):
            for name, tens, okv in (("K", dev.K, kv[0]), ("V", dev.V, kv[1])):
                g = bf16_bits_to_f32(tens[l].cpu().numpy().view(np.uint16))[slots // ps, :, slots % ps, :]
                r = okv[l][slots // ps, :, slots % ps, :]
                e = rel_l2(g, r)
                assert e < HIDDEN_TOL, (tag, name, l, e)
    print(f"[step {tag}] {res}", flush=True)
    return got, ref, res
