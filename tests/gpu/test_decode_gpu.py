"""Decode attention through orthrus_step against the oracle: decode-heavy
batches whose sizes select each decode split length (4096 down to 128 keys
per workgroup; at 4096 every row of these batches is one split, with no
combine), every grouped-query ratio at head dims 64 and 128, page
sizes that do and do not divide the 16-key blocks (5, 7, 16, 32, 64, 128),
and contexts on block and split boundaries.  Weights are drawn wider than the model default
(std 0.05) so that attention is far from uniform and its output is not
lost under the residual stream."""

import numpy as np
import pytest

from synth import model as sm
from synth import workloads as wl
from tests._gpu import make_pair, run_and_compare

pytestmark = pytest.mark.gpu


def decode_batch(cfg, ctxs, n_pages, extra_chunks=(), seed=0):
    """Decode rows at the given contexts, optionally preceded by embedding
    chunks (n_tokens, ctx) with mean pooling into slots 0, 1, ..."""
    rng = np.random.default_rng(seed)
    alloc = wl.PageAllocator(n_pages, seed=seed + 1)
    bb = wl.BatchBuilder(cfg, alloc)
    entries = []
    for j, (n, c) in enumerate(extra_chunks):
        req = bb.add(wl.Request(j, wl.EMBED, list(rng.integers(0, cfg.vocab, c + n)), pool_slot=j,
                                pool_kind=wl.POOL_MEAN))
        req.done = c
        entries.append((j, wl.EMBED, n, c == 0, True))
    for j, c in enumerate(ctxs):
        req = bb.add(wl.Request(1000 + j, wl.DECODE, list(rng.integers(0, cfg.vocab, int(c) + 1))))
        req.done = int(c)
        entries.append((1000 + j, wl.DECODE, 1, 0, 1))
    return bb.build(entries)


def pages_needed(cfg, ctxs, extra_chunks=()):
    ps = cfg.page_size
    return int(sum(-(-(int(c) + 1) // ps) for c in ctxs) + sum(-(-(n + c) // ps) for n, c in extra_chunks)) + 4


def expected_split(cfg, ctxs):
    """The split the library picks: the largest of 4096, 2048, ..., 128 keys
    that still gives 2048 decode workgroups."""
    split = 4096 if cfg.head_dim >= 64 else 128
    while split > 128 and cfg.n_kv_heads * sum((int(c) + split) // split for c in ctxs) < 2048:
        split //= 2
    return split


CASES = [
    # (name, cfg, contexts, embedding chunks)
    ("hd128-g4-ps16-split1024",
     sm.ModelConfig(n_layers=1, d_model=512, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=512,
                    vocab=512, page_size=16, rope_theta=1e6),
     [0, 1, 15, 16, 17, 63, 64, 65, 511, 512, 513, 1023] + list(np.random.default_rng(1).integers(1000, 3000, 130)),
     [(100, 0)]),
    ("hd128-g8-ps16-split128",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=16, n_kv_heads=2, head_dim=128, ffn_dim=256,
                    vocab=300, page_size=16, rope_theta=1e6),
     list(np.random.default_rng(2).integers(300, 1500, 200)) + [127, 128, 129],
     []),
    ("hd64-g1-ps7-split1024",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=8, head_dim=64, ffn_dim=256,
                    vocab=300, page_size=7, rope_theta=1e4),
     list(np.random.default_rng(3).integers(500, 2500, 170)) + [6, 7, 8, 14, 15],
     [(40, 300)]),
    ("hd64-g2-ps32-split256",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=4, head_dim=64, ffn_dim=256,
                    vocab=300, page_size=32, rope_theta=1e4),
     list(np.random.default_rng(4).integers(200, 1200, 160)),
     [(64, 0), (33, 700)]),
    ("hd128-g1-ps16-split256",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=128, ffn_dim=256,
                    vocab=300, page_size=16, rope_theta=1e6),
     list(np.random.default_rng(5).integers(100, 1000, 200)),
     []),
    ("hd128-g2-ps5-split128",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=128, ffn_dim=256,
                    vocab=300, page_size=5, rope_theta=1e6),
     list(np.random.default_rng(6).integers(1, 900, 90)) + [0, 4, 5, 6],
     []),
    # pages of 64 keys (one page per 64-key chunk tile: the page-stride
    # addressing of whole tiles) and of 128 keys (larger than a tile: the
    # per-key form), with embedding chunks at several contexts
    ("hd128-g4-ps64-split128",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=256,
                    vocab=300, page_size=64, rope_theta=1e6),
     list(np.random.default_rng(7).integers(300, 1200, 100)) + [63, 64, 65, 127, 128],
     [(200, 0), (130, 64), (77, 300)]),
    # one workgroup per row and KV head (the boundary contexts 4095 and 4096
    # give one split and two), two splits of 2048 per row, and 512
    ("hd64-g1-ps16-split4096",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=8, head_dim=64, ffn_dim=256,
                    vocab=300, page_size=16, rope_theta=1e6),
     list(np.random.default_rng(9).integers(300, 1800, 254)) + [4095, 4096],
     [(50, 0)]),
    ("hd64-g2-ps32-split2048",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=4, head_dim=64, ffn_dim=256,
                    vocab=300, page_size=32, rope_theta=1e6),
     list(np.random.default_rng(10).integers(2100, 3900, 300)),
     []),
    ("hd128-g4-ps16-split512",
     sm.ModelConfig(n_layers=1, d_model=512, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=512,
                    vocab=512, page_size=16, rope_theta=1e6),
     list(np.random.default_rng(11).integers(1000, 3000, 62)) + [511, 512, 513],
     []),
    ("hd64-g2-ps128-split256",
     sm.ModelConfig(n_layers=1, d_model=256, n_q_heads=8, n_kv_heads=4, head_dim=64, ffn_dim=256,
                    vocab=300, page_size=128, rope_theta=1e4),
     list(np.random.default_rng(8).integers(200, 1500, 150)) + [127, 128, 129, 255, 256],
     [(150, 0), (100, 128), (65, 1000)]),
]


@pytest.mark.parametrize("name,cfg,ctxs,chunks", CASES, ids=[c[0] for c in CASES])
def test_decode_splits(name, cfg, ctxs, chunks):
    want = int(name.rsplit("split", 1)[1])
    assert expected_split(cfg, ctxs) == want, (name, expected_split(cfg, ctxs))
    n_pages = pages_needed(cfg, ctxs, chunks)
    b = decode_batch(cfg, ctxs, n_pages, chunks, seed=len(ctxs))
    bits = sm.make_weights(cfg, seed=7, std=0.05, gain_std=0.1)
    kv = wl.synthetic_kv(cfg, n_pages, seed=3)
    dev, orc = make_pair(cfg, n_pages, bits, kv_bits=kv, max_tokens=max(b.n_tokens, 16),
                         max_items=b.n_items, slots=max(len(chunks), 1))
    print(f"[{name}] rows={b.n_tokens} decode={len(ctxs)} pages={n_pages} split={want}", flush=True)
    run_and_compare(cfg, dev, orc, b, tag=name)
    dev.close()
