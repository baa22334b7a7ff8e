"""Intra-Batch Scheduling and the host step driver (oracle side, pure Python).

Follows "Efficient Iterative Retrieval with Heterogeneous Batching"
(paperpeel full text), §4 Intra-Batch Scheduling: §4.1 (proportional
allocation, per-type FCFS, no head-of-line blocking) and §4.2 Scheduler
Design (decode reservation first; the residual budget filled by alternating
between the embedding and generation queues with token-weighted credit
accumulators; embedding inputs admitted in chunks of at most C tokens);
§3.2 Batch Unit for the order of the emitted batch; §2.2 Generation for the
decode phase (one new token per step, appended to the request's KV).

Readings taken where the page is silent (the same in the C++ scheduler):
 1. Each step first gives one row to every generation request in its
    decode phase, in submission order, while budget remains.  A decode row
    whose position needs a new KV page when none is free waits this step.
 2. The embedding queue and the generation (prompt) queue hold requests with
    input tokens not yet scheduled, in submission order.
 3. The weights w_e and w_g are the queues' unscheduled input tokens at the
    start of the step's fill phase.
 4. Selection: while both queues are open, a_e += w_e and a_g += w_g; the
    embedding queue is taken when a_e >= a_g (ties to embedding), else the
    generation queue; the taken accumulator loses w_e + w_g.  When one queue
    is closed the other is served alone and the accumulators stay as they
    are.  A queue that is empty at the start of a step has its credit reset
    to 0 (credits persist only while the queue is nonempty).
 5. ScheduleOne takes the next request of the chosen queue not yet
    scheduled in this step (FIFO, at most one chunk per request per step).
    Its chunk is min(C, unscheduled tokens), so chunks start at multiples of
    C.  It is admitted only if it fits the residual budget, its KV pages are
    free and, for the first chunk of an embedding request, a pooling slot is
    free; otherwise the queue closes for the step (strict FCFS, no skipping)
    and the accumulator change of that selection is undone.  A queue also
    closes once all its requests are scheduled in this step.
 6. Generation prompts are chunked like embedding inputs; the chunk that
    completes a prompt emits logits.  A generation request with m new tokens
    takes its first token from those logits and then runs m - 1 decode rows.
 7. Pages come from a FIFO free list (given by the caller) and return to its
    back, in the request's page order, when the request finishes; pooling
    slots likewise from 0 .. n_slots-1.
 8. The emitted batch lists embedding chunks, then prompt chunks, then decode
    rows, each group in submission order.
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

EMBED, PREFILL, DECODE = 0, 1, 2


def select(a_e: int, a_g: int, w_e: int, w_g: int):
    """One selection of §4.2 with both queues open: returns (choice, a_e,
    a_g) with choice 0 = embedding, 1 = generation."""
    a_e += w_e
    a_g += w_g
    if a_e >= a_g:
        return 0, a_e - (w_e + w_g), a_g
    return 1, a_e, a_g - (w_e + w_g)


@dataclass
class Req:
    req_id: int
    kind: int                 # EMBED or PREFILL (a generation request)
    tokens: List[int]
    pool_kind: int = 0
    max_new: int = 0
    order: int = 0            # submission index
    done: int = 0             # input tokens scheduled so far (and in KV)
    pages: List[int] = field(default_factory=list)
    slot: int = -1
    produced: int = 0         # generated tokens so far
    pending: int = -1         # generated token the next decode row consumes
    kv: int = 0               # tokens written to the KV cache


class IBSOracle:
    """parity unpinned for the exact batches of a long run: the pages give no
    trace; pinned for the properties §4 states (tests/oracle/test_pins_ibs.py)."""

    def __init__(self, budget: int, chunk: int, page_size: int, free_pages, n_slots: int):
        self.B, self.C, self.ps = int(budget), int(chunk), int(page_size)
        self.free_pages = [int(p) for p in free_pages]
        self.free_slots = list(range(n_slots))
        self.reqs: Dict[int, Req] = {}
        self.emb_q: List[Req] = []
        self.gen_q: List[Req] = []
        self.decoding: List[Req] = []
        self.a_e = 0
        self.a_g = 0
        self.n_sub = 0
        self.last = None          # (items, sched) of the batch awaiting commit

    def submit(self, req_id: int, kind: int, tokens, pool_kind: int = 0, max_new: int = 0) -> None:
        assert kind in (EMBED, PREFILL) and len(tokens) >= 1 and req_id not in self.reqs
        assert kind == EMBED or max_new >= 1
        r = Req(req_id, kind, [int(t) for t in tokens], pool_kind, max_new, self.n_sub)
        self.n_sub += 1
        self.reqs[req_id] = r
        (self.emb_q if kind == EMBED else self.gen_q).append(r)

    def _pages_needed(self, r: Req, upto: int) -> int:
        return max(0, -(-upto // self.ps) - len(r.pages))

    def next(self):
        """Build the next batch: a list of item dicts (fields of
        orthrus_item, pages listed per item) and token ids, or None when no
        work can be scheduled."""
        assert self.last is None, "commit the previous batch first"
        R = self.B
        sched = []   # (kind, req, n_tokens)
        # 1. decode reservation
        for r in sorted(self.decoding, key=lambda q: q.order):
            if R == 0:
                break
            need = self._pages_needed(r, r.kv + 1)
            if need > len(self.free_pages):
                continue
            r.pages.extend(self.free_pages[:need])
            del self.free_pages[:need]
            sched.append((DECODE, r, 1))
            R -= 1
        # 2. fill
        w_e = sum(len(r.tokens) - r.done for r in self.emb_q)
        w_g = sum(len(r.tokens) - r.done for r in self.gen_q)
        if not self.emb_q:
            self.a_e = 0
        if not self.gen_q:
            self.a_g = 0
        nxt = [0, 0]                       # next candidate index per queue
        queues = [self.emb_q, self.gen_q]
        open_ = [bool(self.emb_q), bool(self.gen_q)]
        while R > 0 and (open_[0] or open_[1]):
            saved = (self.a_e, self.a_g)
            if open_[0] and open_[1]:
                pick, self.a_e, self.a_g = select(self.a_e, self.a_g, w_e, w_g)
            else:
                pick = 0 if open_[0] else 1
            q = queues[pick]
            if nxt[pick] >= len(q):
                open_[pick] = False
                self.a_e, self.a_g = saved
                continue
            r = q[nxt[pick]]
            n = min(self.C, len(r.tokens) - r.done)
            need = self._pages_needed(r, r.done + n)
            needs_slot = r.kind == EMBED and r.done == 0
            if n > R or need > len(self.free_pages) or (needs_slot and not self.free_slots):
                open_[pick] = False
                self.a_e, self.a_g = saved
                continue
            r.pages.extend(self.free_pages[:need])
            del self.free_pages[:need]
            if needs_slot:
                r.slot = self.free_slots.pop(0)
            sched.append((r.kind, r, n))
            nxt[pick] += 1
            R -= n
        if not sched:
            return None
        # 3. emit: kind order, then submission order
        sched.sort(key=lambda s: (s[0], s[1].order))
        items, toks, pages = [], [], []
        for kind, r, n in sched:
            if kind == DECODE:
                it = dict(kind=DECODE, req_id=r.req_id, n_tokens=1, ctx_len=r.kv, pool_slot=-1,
                          pool_kind=0, is_first=0, is_last=1)
                toks.append(r.pending)
            else:
                it = dict(kind=kind, req_id=r.req_id, n_tokens=n, ctx_len=r.done,
                          pool_slot=r.slot if kind == EMBED else -1,
                          pool_kind=r.pool_kind if kind == EMBED else 0,
                          is_first=int(kind == EMBED and r.done == 0),
                          is_last=int(r.done + n == len(r.tokens)))
                toks.extend(r.tokens[r.done: r.done + n])
            it["page_off"] = len(pages)
            it["n_pages"] = len(r.pages)
            pages.extend(r.pages)
            items.append(it)
        self.last = (items, sched)
        return items, np.asarray(toks, np.int32), np.asarray(pages, np.int32)

    def _finish(self, r: Req) -> None:
        self.free_pages.extend(r.pages)
        r.pages = []
        if r.slot >= 0:
            self.free_slots.append(r.slot)
            r.slot = -1

    def commit(self, sampled) -> None:
        """Advance after the step ran; sampled[k] is the token taken from
        logit row k (prompt chunks completing their prompt, then decode
        rows, in item order)."""
        items, sched = self.last
        self.last = None
        k = 0
        for kind, r, n in sorted(sched, key=lambda s: (s[0], s[1].order)):
            if kind == DECODE:
                r.kv += 1
                r.produced += 1
                r.pending = int(sampled[k])
                k += 1
                if r.produced == r.max_new:
                    self.decoding.remove(r)
                    self._finish(r)
                continue
            r.done += n
            r.kv = r.done
            if r.done == len(r.tokens):
                (self.emb_q if kind == EMBED else self.gen_q).remove(r)
                if kind == EMBED:
                    self._finish(r)
                else:
                    r.produced = 1
                    r.pending = int(sampled[k])
                    k += 1
                    if r.max_new > 1:
                        self.decoding.append(r)
                    else:
                        self._finish(r)
        assert k == len(sampled), (k, len(sampled))
