// Intra-batch scheduler and host step driver (host C++, no device work).
//
// Efficient Iterative Retrieval with Heterogeneous Batching, §4 Intra-Batch
// Scheduling: every step first reserves one row for each generation
// request in its decode phase, then fills the residual token budget from the
// embedding and generation queues, choosing between them with token-weighted
// credit accumulators (a_e += w_e, a_g += w_g, take the larger, subtract
// w_e + w_g), which converges to the w_e : w_g mix and keeps each backlogged
// queue within one scheduling opportunity of its share; inputs are admitted
// in chunks of at most C tokens, so a backlogged embedding queue leaves
// fewer than C tokens of the budget unused.  §3.2 Batch Unit: the emitted
// batch lists embedding chunks, then prompt chunks, then decode rows.
//
// Where the page is silent the scheduler takes these readings: decode rows
// in submission order, a decode that needs a page when none is free waits;
// weights are the queues' unscheduled input tokens at the start of the fill;
// ties go to the embedding queue; a queue empty at the start of a step has
// its credit reset; the selected queue offers its next request not yet
// scheduled in this step (strict FCFS, one chunk per request per step) and
// closes for the step, with that selection's credit change undone, when the
// chunk does not fit the budget, the free pages or (first embedding chunk)
// the free pooling slots, or when it has no request left; prompts are
// chunked like embedding inputs; a generation request with m new tokens
// takes its first from the logits of the chunk completing its prompt and
// then runs m - 1 decode rows; pages and slots come from FIFO free lists and
// return to their back when a request finishes.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <memory>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/orthrus.h"

namespace {

struct SReq {
  int32_t id = 0, kind = 0, pool_kind = 0, max_new = 0;
  int64_t order = 0;                 // submission index
  std::vector<int32_t> tokens;       // input tokens
  int32_t done = 0;                  // input tokens scheduled (and in the KV cache)
  int32_t slot = -1;                 // pooling slot (embedding)
  int32_t produced = 0;              // generated tokens
  int32_t pending = -1;              // generated token the next decode row consumes
  int32_t kv = 0;                    // tokens in the KV cache
  std::vector<int32_t> pages;
};

struct Sched {
  int32_t kind;
  SReq *r;
  int32_t n;
};

}  // namespace

struct orthrus_sched {
  int32_t B = 0, C = 0, ps = 0;
  std::deque<int32_t> free_pages, free_slots;
  std::unordered_map<int32_t, std::unique_ptr<SReq>> reqs;
  std::unordered_set<int32_t> ids_seen;
  std::vector<SReq *> emb_q, gen_q, decoding;
  int64_t a_e = 0, a_g = 0, n_sub = 0;
  bool pending = false;
  std::vector<Sched> sched;
  std::vector<orthrus_item> items;
  std::vector<int32_t> toks, pages;
};

namespace {

int32_t pages_needed(const orthrus_sched &s, const SReq &r, int64_t upto) {
  const int64_t need = (upto + s.ps - 1) / s.ps - (int64_t)r.pages.size();
  return need > 0 ? (int32_t)need : 0;
}

void take_pages(orthrus_sched &s, SReq &r, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    r.pages.push_back(s.free_pages.front());
    s.free_pages.pop_front();
  }
}

void finish(orthrus_sched &s, SReq &r) {
  for (int32_t p : r.pages) s.free_pages.push_back(p);
  r.pages.clear();
  if (r.slot >= 0) {
    s.free_slots.push_back(r.slot);
    r.slot = -1;
  }
}

bool by_kind_then_order(const Sched &a, const Sched &b) {
  return a.kind != b.kind ? a.kind < b.kind : a.r->order < b.r->order;
}

}  // namespace

extern "C" {

orthrus_status orthrus_sched_create(int32_t token_budget, int32_t chunk, int32_t page_size,
                                    const int32_t *free_pages, int32_t n_free_pages, int32_t n_pool_slots,
                                    orthrus_sched **out) {
  if (!out || token_budget < 1 || chunk < 1 || page_size < 1 || n_free_pages < 0 || n_pool_slots < 0 ||
      (n_free_pages > 0 && !free_pages))
    return ORTHRUS_EINVAL;
  *out = nullptr;
  auto *s = new orthrus_sched();
  s->B = token_budget;
  s->C = chunk;
  s->ps = page_size;
  s->free_pages.assign(free_pages, free_pages + n_free_pages);
  for (int32_t i = 0; i < n_pool_slots; ++i) s->free_slots.push_back(i);
  *out = s;
  return ORTHRUS_OK;
}

void orthrus_sched_destroy(orthrus_sched *s) { delete s; }

orthrus_status orthrus_sched_submit(orthrus_sched *s, int32_t req_id, int32_t kind, const int32_t *tokens,
                                    int32_t n_tokens, int32_t pool_kind, int32_t max_new_tokens) {
  if (!s || !tokens || n_tokens < 1 || (kind != ORTHRUS_EMBED && kind != ORTHRUS_PREFILL)) return ORTHRUS_EINVAL;
  if (kind == ORTHRUS_EMBED && ((pool_kind & ~ORTHRUS_POOL_L2) < ORTHRUS_POOL_MEAN ||
                                (pool_kind & ~ORTHRUS_POOL_L2) > ORTHRUS_POOL_BUFFER))
    return ORTHRUS_EINVAL;
  if (kind == ORTHRUS_PREFILL && max_new_tokens < 1) return ORTHRUS_EINVAL;
  if (s->ids_seen.count(req_id)) return ORTHRUS_EINVAL;
  auto r = std::make_unique<SReq>();
  r->id = req_id;
  r->kind = kind;
  r->pool_kind = kind == ORTHRUS_EMBED ? pool_kind : 0;
  r->max_new = kind == ORTHRUS_PREFILL ? max_new_tokens : 0;
  r->order = s->n_sub++;
  r->tokens.assign(tokens, tokens + n_tokens);
  (kind == ORTHRUS_EMBED ? s->emb_q : s->gen_q).push_back(r.get());
  s->ids_seen.insert(req_id);
  s->reqs[req_id] = std::move(r);
  return ORTHRUS_OK;
}

orthrus_status orthrus_sched_next(orthrus_sched *s, orthrus_batch *out, int32_t *n_logits) {
  if (!s || !out) return ORTHRUS_EINVAL;
  if (s->pending) return ORTHRUS_ESTATE;
  s->sched.clear();
  int64_t R = s->B;
  // 1. decode reservation, submission order
  std::vector<SReq *> dec = s->decoding;
  std::sort(dec.begin(), dec.end(), [](const SReq *a, const SReq *b) { return a->order < b->order; });
  for (SReq *r : dec) {
    if (R == 0) break;
    const int32_t need = pages_needed(*s, *r, (int64_t)r->kv + 1);
    if (need > (int64_t)s->free_pages.size()) continue;
    take_pages(*s, *r, need);
    s->sched.push_back({ORTHRUS_DECODE, r, 1});
    R -= 1;
  }
  // 2. fill the residual budget from the two queues
  int64_t w_e = 0, w_g = 0;
  for (const SReq *r : s->emb_q) w_e += (int64_t)r->tokens.size() - r->done;
  for (const SReq *r : s->gen_q) w_g += (int64_t)r->tokens.size() - r->done;
  if (s->emb_q.empty()) s->a_e = 0;
  if (s->gen_q.empty()) s->a_g = 0;
  std::vector<SReq *> *queues[2] = {&s->emb_q, &s->gen_q};
  size_t nxt[2] = {0, 0};
  bool open[2] = {!s->emb_q.empty(), !s->gen_q.empty()};
  while (R > 0 && (open[0] || open[1])) {
    const int64_t se = s->a_e, sg = s->a_g;
    int pick;
    if (open[0] && open[1]) {
      s->a_e += w_e;
      s->a_g += w_g;
      if (s->a_e >= s->a_g) {
        pick = 0;
        s->a_e -= w_e + w_g;
      } else {
        pick = 1;
        s->a_g -= w_e + w_g;
      }
    } else {
      pick = open[0] ? 0 : 1;
    }
    std::vector<SReq *> &q = *queues[pick];
    if (nxt[pick] >= q.size()) {
      open[pick] = false;
      s->a_e = se;
      s->a_g = sg;
      continue;
    }
    SReq *r = q[nxt[pick]];
    const int32_t n = std::min<int32_t>(s->C, (int32_t)r->tokens.size() - r->done);
    const int32_t need = pages_needed(*s, *r, (int64_t)r->done + n);
    const bool needs_slot = r->kind == ORTHRUS_EMBED && r->done == 0;
    if (n > R || need > (int64_t)s->free_pages.size() || (needs_slot && s->free_slots.empty())) {
      open[pick] = false;
      s->a_e = se;
      s->a_g = sg;
      continue;
    }
    take_pages(*s, *r, need);
    if (needs_slot) {
      r->slot = s->free_slots.front();
      s->free_slots.pop_front();
    }
    s->sched.push_back({r->kind, r, n});
    nxt[pick] += 1;
    R -= n;
  }
  memset(out, 0, sizeof *out);
  if (n_logits) *n_logits = 0;
  if (s->sched.empty()) return ORTHRUS_OK;
  // 3. emit in kind order, then submission order
  std::stable_sort(s->sched.begin(), s->sched.end(), by_kind_then_order);
  s->items.clear();
  s->toks.clear();
  s->pages.clear();
  int32_t nl = 0;
  for (const Sched &e : s->sched) {
    SReq &r = *e.r;
    orthrus_item it{};
    it.kind = e.kind;
    it.req_id = r.id;
    if (e.kind == ORTHRUS_DECODE) {
      it.n_tokens = 1;
      it.ctx_len = r.kv;
      it.pool_slot = -1;
      it.is_last = 1;
      s->toks.push_back(r.pending);
      ++nl;
    } else {
      it.n_tokens = e.n;
      it.ctx_len = r.done;
      it.pool_slot = e.kind == ORTHRUS_EMBED ? r.slot : -1;
      it.pool_kind = e.kind == ORTHRUS_EMBED ? r.pool_kind : 0;
      it.is_first = (e.kind == ORTHRUS_EMBED && r.done == 0) ? 1 : 0;
      it.is_last = (r.done + e.n == (int32_t)r.tokens.size()) ? 1 : 0;
      s->toks.insert(s->toks.end(), r.tokens.begin() + r.done, r.tokens.begin() + r.done + e.n);
      if (e.kind == ORTHRUS_PREFILL && it.is_last) ++nl;
    }
    it.page_off = (int32_t)s->pages.size();
    it.n_pages = (int32_t)r.pages.size();
    s->pages.insert(s->pages.end(), r.pages.begin(), r.pages.end());
    s->items.push_back(it);
  }
  out->n_items = (int32_t)s->items.size();
  out->n_tokens = (int32_t)s->toks.size();
  out->n_page_ids = (int32_t)s->pages.size();
  out->items = s->items.data();
  out->token_ids = s->toks.data();
  out->page_ids = s->pages.data();
  if (n_logits) *n_logits = nl;
  s->pending = true;
  return ORTHRUS_OK;
}

orthrus_status orthrus_sched_commit(orthrus_sched *s, const int32_t *sampled, int32_t n_sampled) {
  if (!s) return ORTHRUS_EINVAL;
  if (!s->pending) return ORTHRUS_ESTATE;
  int32_t need = 0;
  for (const Sched &e : s->sched)
    if (e.kind == ORTHRUS_DECODE || (e.kind == ORTHRUS_PREFILL && e.r->done + e.n == (int32_t)e.r->tokens.size()))
      ++need;
  if (n_sampled != need || (need > 0 && !sampled)) return ORTHRUS_EINVAL;
  int32_t k = 0;
  for (const Sched &e : s->sched) {  // already in kind, then submission order
    SReq &r = *e.r;
    if (e.kind == ORTHRUS_DECODE) {
      r.kv += 1;
      r.produced += 1;
      r.pending = sampled[k++];
      if (r.produced == r.max_new) {
        s->decoding.erase(std::find(s->decoding.begin(), s->decoding.end(), &r));
        finish(*s, r);
      }
      continue;
    }
    r.done += e.n;
    r.kv = r.done;
    if (r.done == (int32_t)r.tokens.size()) {
      std::vector<SReq *> &q = e.kind == ORTHRUS_EMBED ? s->emb_q : s->gen_q;
      q.erase(std::find(q.begin(), q.end(), &r));
      if (e.kind == ORTHRUS_EMBED) {
        finish(*s, r);
      } else {
        r.produced = 1;
        r.pending = sampled[k++];
        if (r.max_new > 1) s->decoding.push_back(&r);
        else finish(*s, r);
      }
    }
  }
  s->sched.clear();
  s->pending = false;
  return ORTHRUS_OK;
}

orthrus_status orthrus_sched_stats(const orthrus_sched *s, int64_t *out8) {
  if (!s || !out8) return ORTHRUS_EINVAL;
  out8[0] = (int64_t)s->emb_q.size();
  out8[1] = (int64_t)s->gen_q.size();
  out8[2] = (int64_t)s->decoding.size();
  out8[3] = (int64_t)s->free_pages.size();
  out8[4] = (int64_t)s->free_slots.size();
  out8[5] = s->a_e;
  out8[6] = s->a_g;
  out8[7] = s->pending ? 1 : 0;
  return ORTHRUS_OK;
}

}  // extern "C"
