"""Seeded synthetic batches: items, token ids, page lists and prior state.

A batch is a list of items sorted by kind (embedding chunks, then
generation prefill chunks, then decode rows) with their token ids laid out
in item order, and a flat list of KV page ids into which each item indexes
with (page_off, n_pages).  Pages are handed out by a FIFO free list that
starts as a seeded permutation of [0, n_pages), so page tables are not
contiguous.  Seeds: weights 0, token ids 1, lengths/contexts 2,
synthetic KV and prior pooling state 3, page permutation 4.
"""

from dataclasses import dataclass, field, astuple
from typing import Dict, List, Optional
import collections

import numpy as np

from .model import ModelConfig, TINY, MISTRAL_7B

EMBED, PREFILL, DECODE = 0, 1, 2
POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST, POOL_BUFFER = 0, 1, 2, 3, 4
POOL_L2 = 8   # OR-ed into a pool kind: unit-length output

ITEM_FIELDS = ("kind", "req_id", "n_tokens", "ctx_len", "page_off", "n_pages",
               "pool_slot", "pool_kind", "is_first", "is_last")


@dataclass
class Item:
    kind: int
    req_id: int
    n_tokens: int
    ctx_len: int
    page_off: int = 0
    n_pages: int = 0
    pool_slot: int = -1
    pool_kind: int = 0
    is_first: int = 0
    is_last: int = 0

    def as_tuple(self):
        return astuple(self)


@dataclass
class Batch:
    items: List[Item]
    token_ids: np.ndarray          # int32 [n_tokens], item order
    page_ids: np.ndarray           # int32, items index it with page_off/n_pages

    @property
    def n_items(self) -> int:
        return len(self.items)

    @property
    def n_tokens(self) -> int:
        return int(self.token_ids.shape[0])

    def items_array(self) -> np.ndarray:
        if not self.items:
            return np.zeros((0, len(ITEM_FIELDS)), np.int32)
        return np.array([it.as_tuple() for it in self.items], dtype=np.int32)

    def item_pages(self, i: int) -> np.ndarray:
        it = self.items[i]
        return self.page_ids[it.page_off: it.page_off + it.n_pages]


class PageAllocator:
    """FIFO free list over [0, n_pages), initialised to a seeded permutation."""

    def __init__(self, n_pages: int, seed: int = 4):
        perm = np.random.default_rng(seed).permutation(n_pages)
        self.free = collections.deque(int(p) for p in perm)
        self.n_pages = n_pages

    def alloc(self, k: int) -> List[int]:
        if k > len(self.free):
            raise MemoryError(f"page pool exhausted: need {k}, have {len(self.free)}")
        return [self.free.popleft() for _ in range(k)]

    def release(self, pages: List[int]) -> None:
        self.free.extend(pages)


@dataclass
class Request:
    req_id: int
    kind: int                       # EMBED or generation (PREFILL/DECODE)
    tokens: List[int]               # all tokens known so far
    pages: List[int] = field(default_factory=list)
    done: int = 0                   # tokens already in the KV cache
    pool_slot: int = -1
    pool_kind: int = POOL_MEAN


class BatchBuilder:
    """Assembles batches from requests, growing each request's page list."""

    def __init__(self, cfg: ModelConfig, allocator: PageAllocator):
        self.cfg = cfg
        self.alloc = allocator
        self.reqs: Dict[int, Request] = {}

    def add(self, req: Request) -> Request:
        self.reqs[req.req_id] = req
        return req

    def _ensure_pages(self, req: Request, upto: int) -> None:
        need = -(-upto // self.cfg.page_size)
        if need > len(req.pages):
            req.pages.extend(self.alloc.alloc(need - len(req.pages)))

    def build(self, entries) -> Batch:
        """entries: (req_id, kind, n_tokens, is_first, is_last) tuples, kind-sorted."""
        items, toks, pages = [], [], []
        for req_id, kind, n, first, last in entries:
            req = self.reqs[req_id]
            c = req.done
            self._ensure_pages(req, c + n)
            it = Item(kind=kind, req_id=req_id, n_tokens=n, ctx_len=c,
                      page_off=len(pages), n_pages=len(req.pages),
                      pool_slot=req.pool_slot if kind == EMBED else -1,
                      pool_kind=req.pool_kind if kind == EMBED else 0,
                      is_first=int(first), is_last=int(last))
            pages.extend(req.pages)
            toks.extend(req.tokens[c: c + n])
            items.append(it)
        return Batch(items, np.asarray(toks, np.int32).reshape(-1),
                     np.asarray(pages, np.int32).reshape(-1))

    def commit(self, batch: Batch) -> None:
        """Advance request state after the step ran; free finished embeddings."""
        for it in batch.items:
            req = self.reqs[it.req_id]
            req.done += it.n_tokens
            if it.kind == EMBED and it.is_last:
                self.alloc.release(req.pages)
                req.pages = []


def tiny_workload(seed_tok: int = 1, cfg: ModelConfig = TINY, pool_kind: int = POOL_MEAN,
                  chunk: int = 16, n_pages: int = 64):
    """Small correctness workload: generation prompts of 30 and 50 tokens are
    prefilled first; then three mixed steps run two embedding requests of 40
    and 24 tokens in chunks of 16 beside one decode row per generation
    request (contexts 30 and 50 at the first mixed step).

    Returns (cfg, batches, n_pages).  Decode tokens are seeded, not sampled.
    """
    rng = np.random.default_rng(seed_tok)
    V = cfg.vocab
    alloc = PageAllocator(n_pages, seed=4)
    bb = BatchBuilder(cfg, alloc)
    gen_len = {100: 30, 101: 50}
    for rid, n in gen_len.items():
        bb.add(Request(rid, PREFILL, list(rng.integers(0, V, n + 3))))
    emb_len = {0: 40, 1: 24}
    for slot, (rid, n) in enumerate(emb_len.items()):
        bb.add(Request(rid, EMBED, list(rng.integers(0, V, n)), pool_slot=slot,
                       pool_kind=pool_kind))
    batches = []
    b = bb.build([(100, PREFILL, 30, 1, 1), (101, PREFILL, 50, 1, 1)])
    batches.append(b)
    bb.commit(b)
    for s in range(3):
        entries = []
        for rid, n in emb_len.items():
            done = bb.reqs[rid].done
            if done >= n:
                continue
            c = min(chunk, n - done)
            entries.append((rid, EMBED, c, done == 0, done + c == n))
        entries += [(100, DECODE, 1, 0, 1), (101, DECODE, 1, 0, 1)]
        b = bb.build(entries)
        batches.append(b)
        bb.commit(b)
    return cfg, batches, n_pages


def one_layer_workload(seed_len: int = 2, seed_tok: int = 1,
                       cfg: ModelConfig = None, n_embed: int = 8, embed_len: int = 512,
                       n_decode: int = 64, ctx_lo: int = 500, ctx_hi: int = 3500,
                       pool_kind: int = POOL_LAST):
    """One Mistral-7B-shaped layer: 8 embedding chunks of 512 tokens (first and
    last chunk of their request, last-token pooling) and 64 decode rows with
    KV contexts uniform in [500, 3500], KV pages of 16.

    Returns (cfg, batch, n_pages).  The decode contexts are prior KV whose
    values the caller fills with seeded synthetic data.
    """
    if cfg is None:
        cfg = MISTRAL_7B.with_(n_layers=1)
    rl = np.random.default_rng(seed_len)
    rt = np.random.default_rng(seed_tok)
    ctxs = rl.integers(ctx_lo, ctx_hi + 1, n_decode)
    ps = cfg.page_size
    n_pages = n_embed * (-(-embed_len // ps)) + int(sum(-(-(int(c) + 1) // ps) for c in ctxs))
    alloc = PageAllocator(n_pages, seed=4)
    bb = BatchBuilder(cfg, alloc)
    entries = []
    for i in range(n_embed):
        bb.add(Request(i, EMBED, list(rt.integers(0, cfg.vocab, embed_len)),
                       pool_slot=i, pool_kind=pool_kind))
        entries.append((i, EMBED, embed_len, 1, 1))
    for j, c in enumerate(ctxs):
        rid = 1000 + j
        req = bb.add(Request(rid, DECODE, list(rt.integers(0, cfg.vocab, int(c) + 1))))
        req.done = int(c)
        entries.append((rid, DECODE, 1, 0, 1))
    batch = bb.build(entries)
    return cfg, batch, n_pages


def random_batch(cfg: ModelConfig, seed: int, max_items: int = 12, max_len: int = 40,
                 max_ctx: int = 70, n_pages: Optional[int] = None, n_slots: int = 16,
                 pool_kinds=(POOL_MEAN, POOL_WMEAN, POOL_CLS, POOL_LAST)):
    """A random valid ragged batch (for packer and attention coverage tests);
    embedding items draw their pool kind from ``pool_kinds``."""
    rng = np.random.default_rng(seed)
    ps = cfg.page_size
    n_e, n_p, n_d = (int(x) for x in rng.integers(0, max_items // 3 + 1, 3))
    if n_e + n_p + n_d == 0:
        n_d = 1
    kinds = [EMBED] * n_e + [PREFILL] * n_p + [DECODE] * n_d
    specs = []
    slots = list(rng.permutation(n_slots)[:n_e])
    for k in kinds:
        n = 1 if k == DECODE else int(rng.integers(1, max_len + 1))
        c = int(rng.integers(0, max_ctx + 1))
        first = 0
        if k == EMBED:
            first = int(rng.integers(0, 2))
            if first:
                c = 0
        specs.append((k, n, c, first))
    need = sum(-(-(c + n) // ps) for _, n, c, _ in specs)
    if n_pages is None:
        n_pages = need + int(rng.integers(0, 8))
    alloc = PageAllocator(n_pages, seed=seed + 7)
    items, toks, pages = [], [], []
    for idx, (k, n, c, first) in enumerate(specs):
        pg = alloc.alloc(-(-(c + n) // ps))
        it = Item(kind=k, req_id=int(idx * 3 + 5), n_tokens=n, ctx_len=c,
                  page_off=len(pages), n_pages=len(pg),
                  pool_slot=int(slots[idx]) if k == EMBED else -1,
                  pool_kind=int(pool_kinds[int(rng.integers(0, len(pool_kinds)))]) if k == EMBED else 0,
                  is_first=first, is_last=int(rng.integers(0, 2)) if k != DECODE else 1)
        pages.extend(pg)
        toks.extend(int(t) for t in rng.integers(0, cfg.vocab, n))
        items.append(it)
    return Batch(items, np.asarray(toks, np.int32).reshape(-1),
                 np.asarray(pages, np.int32).reshape(-1)), n_pages


def kv_pool_shape(cfg: ModelConfig, n_pages: int):
    """K (and V) cache layout: [layer][page][kv_head][slot_in_page][head_dim]."""
    return (cfg.n_layers, n_pages, cfg.n_kv_heads, cfg.page_size, cfg.head_dim)


def synthetic_kv(cfg: ModelConfig, n_pages: int, seed: int = 3):
    """Seeded prior KV content (unit normal) for the whole pool, as uint16 bf16 bits."""
    from .model import normal_bf16
    shape = kv_pool_shape(cfg, n_pages)
    n = int(np.prod(shape))
    k = normal_bf16([seed, 0], n, 1.0).reshape(shape)
    v = normal_bf16([seed, 1], n, 1.0).reshape(shape)
    return k, v


# ---- the three large workloads ----------------------------------------------
# Prior state of a workload: every KV page of every layer holds SplitMix64
# values (seed KV_SEED, tensor 0 for K and 1 for V) over the linear index of
# the [layer][page][kv_head][slot][head_dim] pool; pooling slots hold
# SplitMix64 values (tensor 2 for the running sum, 3 for the kept state) over
# slot * d + j, and a weight total equal to the closed form of the tokens
# before the chunk (c for mean, c(c+1)/2 for weighted mean).
KV_SEED = 3
POOL_SUM_TID, POOL_KEPT_TID = 2, 3


@dataclass
class Workload:
    cfg: ModelConfig
    batches: List[Batch]
    n_pages: int
    n_slots: int
    prior_wsum: Dict[int, float] = field(default_factory=dict)   # slot -> weight total before step 0


def _prior_total(kind: int, c: int) -> float:
    if kind == POOL_MEAN:
        return float(c)
    if kind == POOL_WMEAN:
        return float(c * (c + 1) // 2)
    return 0.0


def _budget_batch(cfg, rng_tok, bb, emb_entries, dec_ids):
    return bb.build(emb_entries + [(rid, DECODE, 1, 0, 1) for rid in dec_ids])


def nine_to_one_workload(n_layers: int = 32, steps: int = 10, budget: int = 8192, chunk: int = 256,
                         seed_len: int = 2, seed_tok: int = 1, n_decode: int = 819,
                         cfg: ModelConfig = None) -> Workload:
    """Mistral-7B shape at a 9:1 embedding:generation token mix: 819 decode
    rows (contexts uniform in [500, 3500], +1 per step) and embedding
    requests of U[256, 4096] tokens in chunks of 256 with mean pooling,
    admitted first come first served into the remaining budget of 8192
    tokens (at most one chunk per request per step; a chunk is admitted only
    when it fits), for `steps` consecutive steps with pooling state and KV
    carried between steps.  LoRA rank 16."""
    cfg = (cfg or MISTRAL_7B).with_(n_layers=n_layers, lora_rank=16)
    rl = np.random.default_rng(seed_len)
    rt = np.random.default_rng(seed_tok)
    ps = cfg.page_size
    ctxs = rl.integers(500, 3501, n_decode)
    emb_lens = list(rl.integers(256, 4097, 400))
    dec_pages = int(sum(-(-(int(c) + steps) // ps) for c in ctxs))
    emb_pages = (budget // chunk + 2) * (-(-(steps * chunk) // ps)) + 64
    n_pages = dec_pages + emb_pages
    alloc = PageAllocator(n_pages, seed=4)
    bb = BatchBuilder(cfg, alloc)
    dec_ids = []
    for j, c in enumerate(ctxs):
        rid = 100000 + j
        req = bb.add(Request(rid, DECODE, list(rt.integers(0, cfg.vocab, int(c) + steps + 1))))
        req.done = int(c)
        dec_ids.append(rid)
    n_slots = budget // chunk + 2
    free_slots = collections.deque(range(n_slots))
    queue = collections.deque(range(len(emb_lens)))
    active = []  # request ids in arrival order
    lens = {}
    batches = []
    for _ in range(steps):
        room = budget - len(dec_ids)
        entries = []
        # active requests first (arrival order), then admit new ones
        for rid in list(active):
            n = lens[rid]
            done = bb.reqs[rid].done
            c = min(chunk, n - done)
            if c <= room:
                entries.append((rid, EMBED, c, done == 0, done + c == n))
                room -= c
        while queue and room >= min(chunk, emb_lens[queue[0]]) and free_slots:
            i = queue.popleft()
            rid = i
            n = int(emb_lens[i])
            lens[rid] = n
            bb.add(Request(rid, EMBED, list(rt.integers(0, cfg.vocab, n)), pool_slot=free_slots.popleft(),
                           pool_kind=POOL_MEAN))
            active.append(rid)
            c = min(chunk, n)
            entries.append((rid, EMBED, c, True, c == n))
            room -= c
        b = _budget_batch(cfg, rt, bb, entries, dec_ids)
        batches.append(b)
        bb.commit(b)
        for it in b.items:
            if it.kind == EMBED and it.is_last:
                active.remove(it.req_id)
                free_slots.append(bb.reqs[it.req_id].pool_slot)
    return Workload(cfg, batches, n_pages, n_slots)


def five_to_five_workload(n_layers: int = 32, seed_len: int = 2, seed_tok: int = 1,
                          cfg: ModelConfig = None) -> Workload:
    """Mistral-7B shape at a 5:5 mix, LoRA rank 64: four embedding requests of
    4096 tokens at chunk indices 0..3 of a 1024 chunking with position-
    weighted mean pooling (the later chunks carry synthetic prior state),
    seven 500-token prompt prefill chunks and 596 decode rows with contexts
    uniform in [500, 3500]: 8192 rows."""
    cfg = (cfg or MISTRAL_7B).with_(n_layers=n_layers, lora_rank=64)
    rl = np.random.default_rng(seed_len)
    rt = np.random.default_rng(seed_tok)
    ps = cfg.page_size
    ctxs = rl.integers(500, 3501, 596)
    n_pages = 4 * (4096 // ps) + 7 * (-(-500 // ps)) + int(sum(-(-(int(c) + 1) // ps) for c in ctxs)) + 16
    alloc = PageAllocator(n_pages, seed=4)
    bb = BatchBuilder(cfg, alloc)
    entries, prior = [], {}
    for i in range(4):
        req = bb.add(Request(i, EMBED, list(rt.integers(0, cfg.vocab, 4096)), pool_slot=i, pool_kind=POOL_WMEAN))
        req.done = i * 1024
        prior[i] = _prior_total(POOL_WMEAN, req.done)
        entries.append((i, EMBED, 1024, i == 0, i == 3))
    for k in range(7):
        bb.add(Request(1000 + k, PREFILL, list(rt.integers(0, cfg.vocab, 500))))
        entries.append((1000 + k, PREFILL, 500, True, True))
    for j, c in enumerate(ctxs):
        req = bb.add(Request(100000 + j, DECODE, list(rt.integers(0, cfg.vocab, int(c) + 1))))
        req.done = int(c)
        entries.append((100000 + j, DECODE, 1, 0, 1))
    return Workload(cfg, [bb.build(entries)], n_pages, 4, prior)


def one_to_nine_workload(n_layers: int = 32, budget: int = 8192, seed_len: int = 2, seed_tok: int = 1,
                         cfg: ModelConfig = None) -> Workload:
    """Llama-3.1-8B shape at a decode-heavy 1:9 request mix: 256 decode rows
    with contexts uniform in [500, 3500] reserved first, then embedding
    requests of n_docs ~ U{1..10} x 512 tokens with CLS pooling in chunks of
    512, each at a uniform chunk index (earlier chunks' KV and kept state
    synthetic), filling the 8192-token budget: 15 chunks, 7936 rows."""
    from .model import LLAMA31_8B
    cfg = (cfg or LLAMA31_8B).with_(n_layers=n_layers, lora_rank=16)
    rl = np.random.default_rng(seed_len)
    rt = np.random.default_rng(seed_tok)
    ps = cfg.page_size
    ctxs = rl.integers(500, 3501, 256)
    n_chunks = (budget - 256) // 512
    docs = rl.integers(1, 11, n_chunks)
    idxs = [int(rl.integers(0, d)) for d in docs]
    n_pages = int(sum(-(-(int(c) + 1) // ps) for c in ctxs)) + int(sum(int(d) * 512 // ps for d in docs)) + 16
    alloc = PageAllocator(n_pages, seed=4)
    bb = BatchBuilder(cfg, alloc)
    entries = []
    for i, (d, k) in enumerate(zip(docs, idxs)):
        n = int(d) * 512
        req = bb.add(Request(i, EMBED, list(rt.integers(0, cfg.vocab, n)), pool_slot=i, pool_kind=POOL_CLS))
        req.done = k * 512
        entries.append((i, EMBED, 512, k == 0, (k + 1) * 512 == n))
    for j, c in enumerate(ctxs):
        req = bb.add(Request(100000 + j, DECODE, list(rt.integers(0, cfg.vocab, int(c) + 1))))
        req.done = int(c)
        entries.append((100000 + j, DECODE, 1, 0, 1))
    return Workload(cfg, [bb.build(entries)], n_pages, n_chunks)
