"""Shared test helpers: seeded models and batches run through the oracle."""

import numpy as np

from synth import model as sm
from synth import workloads as wl
from synth.workloads import Item, Batch, PageAllocator, BatchBuilder, Request
import oracle


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def row_rel_l2(a, b):
    """rel-L2 of every row (first axis) of a against b."""
    a = np.asarray(a, np.float64).reshape(len(a), -1)
    b = np.asarray(b, np.float64).reshape(len(b), -1)
    return np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


MINI = sm.ModelConfig(n_layers=4, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                      ffn_dim=256, vocab=512, lora_rank=8, page_size=16, rope_theta=1e4)


class OracleRunner:
    """Holds widened weights, KV pools and pool state for multi-step oracle runs."""

    def __init__(self, cfg, n_pages, dtype=np.float64, seed=0, gain_std=0.1, n_slots=16,
                 weights=None):
        self.cfg = cfg
        self.dtype = dtype
        bits = weights if weights is not None else sm.make_weights(cfg, seed=seed, gain_std=gain_std)
        self.bits = bits
        self.W = oracle.widen_weights(bits, dtype)
        self.kv = oracle.new_kv(cfg, n_pages, dtype)
        self.pool = oracle.new_pool(n_slots, cfg.d_model, dtype)

    def step(self, batch):
        return oracle.step(self.cfg, self.W, batch, self.kv, self.pool, self.dtype)


def single_request_batches(cfg, tokens, chunk, kind=wl.EMBED, pool_kind=wl.POOL_MEAN,
                           slot=0, n_pages=None, seed=4, req_id=7):
    """Chunk one request into batches of one item each."""
    n = len(tokens)
    if n_pages is None:
        n_pages = -(-n // cfg.page_size) + 2
    alloc = PageAllocator(n_pages, seed=seed)
    bb = BatchBuilder(cfg, alloc)
    bb.add(Request(req_id, kind, list(tokens), pool_slot=slot, pool_kind=pool_kind))
    out = []
    done = 0
    while done < n:
        c = min(chunk, n - done)
        b = bb.build([(req_id, kind, c, done == 0, done + c == n)])
        out.append(b)
        bb.commit(b) if kind != wl.EMBED else _commit_keep(bb, b)
        done += c
    return out, n_pages


def _commit_keep(bb, b):
    for it in b.items:
        bb.reqs[it.req_id].done += it.n_tokens
