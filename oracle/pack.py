"""Batch validation and packing metadata (oracle side, pure Python).

Follows "Efficient Iterative Retrieval with Heterogeneous Batching"
(paperpeel full text), §3.2 Batch Unit: a batch holds embedding chunks,
generation prefill chunks and single-token decode rows, sorted by request
type so that each output stage works on a contiguous slice of rows; and
§2.2 (Generation): every processed token appends its KV entries.

Readings taken where the page is silent: kinds are ordered embedding,
prefill, decode; rows follow item order; a token at position p of a request
whose page list is P lives in KV slot P[p // page_size] * page_size +
p % page_size; logits are produced for the last row of a prefill chunk that
completes its prompt and for every decode row, in item order.

Validation checks run in a fixed order and the first failure wins; the C++
packer uses the same order, so status codes compare exactly.
"""

from dataclasses import dataclass
from typing import Dict

import numpy as np

OK, EINVAL, ENOPAGES, ECAPACITY, ESTATE = 0, 1, 2, 3, 4
EMBED, PREFILL, DECODE = 0, 1, 2


class PackError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


@dataclass
class Limits:
    n_pages: int
    max_tokens: int
    max_items: int
    max_pool_slots: int


def pack_py(cfg, batch, limits: Limits) -> Dict[str, np.ndarray]:
    """Validate ``batch`` and return its int32 metadata arrays.

    Keys: cu_q [n+1], pos [T], slot [T], row_item [T], logit_rows [G],
    pool_segs [E, 8] = (row_start, n_rows, pool_slot, pool_kind, is_first,
    is_last, ctx_len, out_index or -1), and the scalar counts n_embed_rows,
    n_prefill_rows, n_decode_rows, n_logits, n_emb.
    Raises PackError(code) on invalid input.
    """
    items = batch.items
    n = len(items)
    T = int(batch.token_ids.shape[0])
    ps = cfg.page_size
    n_ids = int(batch.page_ids.shape[0])
    if n > limits.max_items or T > limits.max_tokens:
        raise PackError(ECAPACITY, "batch exceeds max_items/max_tokens")
    prev = -1
    total = 0
    for i, it in enumerate(items):
        if it.kind not in (EMBED, PREFILL, DECODE):
            raise PackError(EINVAL, f"item {i}: bad kind")
        if it.kind < prev:
            raise PackError(EINVAL, f"item {i}: kinds not sorted")
        prev = it.kind
        if it.n_tokens < 1 or (it.kind == DECODE and it.n_tokens != 1):
            raise PackError(EINVAL, f"item {i}: bad n_tokens")
        if it.ctx_len < 0:
            raise PackError(EINVAL, f"item {i}: negative ctx_len")
        if it.page_off < 0 or it.n_pages < 0 or it.page_off + it.n_pages > n_ids:
            raise PackError(EINVAL, f"item {i}: page range outside page_ids")
        if it.n_pages * ps < it.ctx_len + it.n_tokens:
            raise PackError(ENOPAGES, f"item {i}: too few pages")
        for p in batch.page_ids[it.page_off: it.page_off + it.n_pages]:
            if p < 0 or p >= limits.n_pages:
                raise PackError(ENOPAGES, f"item {i}: page id out of range")
        if it.is_first not in (0, 1) or it.is_last not in (0, 1):
            raise PackError(EINVAL, f"item {i}: flags must be 0/1")
        if it.kind == EMBED:
            if it.pool_slot < 0 or it.pool_slot >= limits.max_pool_slots:
                raise PackError(ESTATE, f"item {i}: pool slot out of range")
            if it.pool_kind & ~8 not in (0, 1, 2, 3, 4):      # a base kind, optionally | L2 (8)
                raise PackError(EINVAL, f"item {i}: bad pool kind")
            if it.is_first and it.ctx_len != 0:
                raise PackError(ESTATE, f"item {i}: first chunk must start at position 0")
        total += it.n_tokens
    if total != T:
        raise PackError(EINVAL, "sum of item lengths differs from token count")
    seen = set()
    for i, it in enumerate(items):
        if it.req_id in seen:
            raise PackError(EINVAL, f"item {i}: request appears twice")
        seen.add(it.req_id)
    seen = set()
    for i, it in enumerate(items):
        if it.kind == EMBED:
            if it.pool_slot in seen:
                raise PackError(ESTATE, f"item {i}: pool slot used twice")
            seen.add(it.pool_slot)
    for t in batch.token_ids:
        if t < 0 or t >= cfg.vocab:
            raise PackError(EINVAL, "token id out of range")

    cu_q = np.zeros(n + 1, np.int32)
    pos = np.zeros(T, np.int32)
    slot = np.zeros(T, np.int32)
    row_item = np.zeros(T, np.int32)
    logit_rows, segs = [], []
    counts = [0, 0, 0]
    n_emb = 0
    r = 0
    for i, it in enumerate(items):
        cu_q[i] = r
        pages = batch.page_ids[it.page_off: it.page_off + it.n_pages]
        for j in range(it.n_tokens):
            p = it.ctx_len + j
            pos[r + j] = p
            slot[r + j] = int(pages[p // ps]) * ps + p % ps
            row_item[r + j] = i
        counts[it.kind] += it.n_tokens
        if it.kind == PREFILL and it.is_last:
            logit_rows.append(r + it.n_tokens - 1)
        elif it.kind == DECODE:
            logit_rows.append(r)
        if it.kind == EMBED:
            out = -1
            if it.is_last:
                out = n_emb
                n_emb += 1
            segs.append((r, it.n_tokens, it.pool_slot, it.pool_kind, it.is_first,
                         it.is_last, it.ctx_len, out))
        r += it.n_tokens
    cu_q[n] = r
    if len(set(slot.tolist())) != T:
        raise PackError(EINVAL, "two rows write the same KV slot")
    return {
        "cu_q": cu_q, "pos": pos, "slot": slot, "row_item": row_item,
        "logit_rows": np.asarray(logit_rows, np.int32),
        "pool_segs": np.asarray(segs, np.int32).reshape(-1, 8),
        "n_embed_rows": counts[EMBED], "n_prefill_rows": counts[PREFILL],
        "n_decode_rows": counts[DECODE], "n_logits": len(logit_rows), "n_emb": n_emb,
    }
