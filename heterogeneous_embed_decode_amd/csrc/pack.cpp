// Host-side validation and packing of a heterogeneous batch.
//
// Rules (Efficient Iterative Retrieval with Heterogeneous Batching, §3.2
// Batch Unit; §2.2 Generation): items arrive sorted by type — embedding
// chunks, then prefill chunks, then single-token decode rows — so each
// output stage reads a contiguous slice of rows; every row appends its K/V
// at the slot of its position in the request's page list.  Checks run in a
// fixed order and the first failure is reported.
#include <cstdio>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "orthrus_internal.h"

namespace orthrus {

static orthrus_status fail(char *err, int32_t len, orthrus_status code, const char *fmt, int a) {
  if (err && len > 0) snprintf(err, (size_t)len, fmt, a);
  return code;
}

orthrus_status validate_and_pack(const orthrus_model_cfg &cfg, const orthrus_batch &b,
                                 HostPack &p, char *err, int32_t elen) {
  const int n = b.n_items, T = b.n_tokens, ps = cfg.page_size;
  if (n < 0 || T < 0 || b.n_page_ids < 0) return fail(err, elen, ORTHRUS_EINVAL, "negative count %d", 0);
  if ((n > 0 && !b.items) || (T > 0 && !b.token_ids) || (b.n_page_ids > 0 && !b.page_ids))
    return fail(err, elen, ORTHRUS_EINVAL, "null batch array %d", 0);
  if (n > cfg.max_items || T > cfg.max_tokens)
    return fail(err, elen, ORTHRUS_ECAPACITY, "batch exceeds max_items/max_tokens (%d)", n);
  int prev = -1;
  long total = 0;
  for (int i = 0; i < n; ++i) {
    const orthrus_item &it = b.items[i];
    if (it.kind < ORTHRUS_EMBED || it.kind > ORTHRUS_DECODE)
      return fail(err, elen, ORTHRUS_EINVAL, "item %d: bad kind", i);
    if (it.kind < prev) return fail(err, elen, ORTHRUS_EINVAL, "item %d: kinds not sorted", i);
    prev = it.kind;
    if (it.n_tokens < 1 || (it.kind == ORTHRUS_DECODE && it.n_tokens != 1))
      return fail(err, elen, ORTHRUS_EINVAL, "item %d: bad n_tokens", i);
    if (it.ctx_len < 0) return fail(err, elen, ORTHRUS_EINVAL, "item %d: negative ctx_len", i);
    if (it.page_off < 0 || it.n_pages < 0 || (long)it.page_off + it.n_pages > b.n_page_ids)
      return fail(err, elen, ORTHRUS_EINVAL, "item %d: page range outside page_ids", i);
    if ((long)it.n_pages * ps < (long)it.ctx_len + it.n_tokens)
      return fail(err, elen, ORTHRUS_ENOPAGES, "item %d: too few pages", i);
    for (int k = 0; k < it.n_pages; ++k) {
      int pg = b.page_ids[it.page_off + k];
      if (pg < 0 || pg >= cfg.n_pages)
        return fail(err, elen, ORTHRUS_ENOPAGES, "item %d: page id out of range", i);
    }
    if ((it.is_first != 0 && it.is_first != 1) || (it.is_last != 0 && it.is_last != 1))
      return fail(err, elen, ORTHRUS_EINVAL, "item %d: flags must be 0/1", i);
    if (it.kind == ORTHRUS_EMBED) {
      if (it.pool_slot < 0 || it.pool_slot >= cfg.max_pool_slots)
        return fail(err, elen, ORTHRUS_ESTATE, "item %d: pool slot out of range", i);
      if ((it.pool_kind & ~ORTHRUS_POOL_L2) < ORTHRUS_POOL_MEAN || (it.pool_kind & ~ORTHRUS_POOL_L2) > ORTHRUS_POOL_BUFFER)
        return fail(err, elen, ORTHRUS_EINVAL, "item %d: bad pool kind", i);
      if (it.is_first && it.ctx_len != 0)
        return fail(err, elen, ORTHRUS_ESTATE, "item %d: first chunk must start at position 0", i);
    }
    total += it.n_tokens;
  }
  if (total != T) return fail(err, elen, ORTHRUS_EINVAL, "sum of item lengths differs from token count %d", T);
  {
    std::unordered_set<int> seen;
    for (int i = 0; i < n; ++i)
      if (!seen.insert(b.items[i].req_id).second)
        return fail(err, elen, ORTHRUS_EINVAL, "item %d: request appears twice", i);
  }
  {
    std::unordered_set<int> seen;
    for (int i = 0; i < n; ++i)
      if (b.items[i].kind == ORTHRUS_EMBED && !seen.insert(b.items[i].pool_slot).second)
        return fail(err, elen, ORTHRUS_ESTATE, "item %d: pool slot used twice", i);
  }
  for (int t = 0; t < T; ++t)
    if (b.token_ids[t] < 0 || b.token_ids[t] >= cfg.vocab)
      return fail(err, elen, ORTHRUS_EINVAL, "token id out of range at row %d", t);

  p.n_items = n;
  p.n_tokens = T;
  p.cu_q.assign(n + 1, 0);
  p.pos.assign(T, 0);
  p.slot.assign(T, 0);
  p.row_item.assign(T, 0);
  p.logit_rows.clear();
  p.pool_segs.clear();
  p.rows_by_kind[0] = p.rows_by_kind[1] = p.rows_by_kind[2] = 0;
  p.n_emb = 0;
  int r = 0;
  for (int i = 0; i < n; ++i) {
    const orthrus_item &it = b.items[i];
    p.cu_q[i] = r;
    const int32_t *pages = b.page_ids + it.page_off;
    for (int j = 0; j < it.n_tokens; ++j) {
      const int pos = it.ctx_len + j;
      p.pos[r + j] = pos;
      p.slot[r + j] = pages[pos / ps] * ps + pos % ps;
      p.row_item[r + j] = i;
    }
    p.rows_by_kind[it.kind] += it.n_tokens;
    if (it.kind == ORTHRUS_PREFILL && it.is_last) p.logit_rows.push_back(r + it.n_tokens - 1);
    else if (it.kind == ORTHRUS_DECODE) p.logit_rows.push_back(r);
    if (it.kind == ORTHRUS_EMBED) {
      int out = -1;
      if (it.is_last) out = p.n_emb++;
      const int32_t seg[8] = {r, it.n_tokens, it.pool_slot, it.pool_kind, it.is_first,
                              it.is_last, it.ctx_len, out};
      p.pool_segs.insert(p.pool_segs.end(), seg, seg + 8);
    }
    r += it.n_tokens;
  }
  p.cu_q[n] = r;
  {
    std::unordered_set<int> seen;
    seen.reserve((size_t)T * 2);
    for (int t = 0; t < T; ++t)
      if (!seen.insert(p.slot[t]).second)
        return fail(err, elen, ORTHRUS_EINVAL, "two rows write the same KV slot (row %d)", t);
  }
  return ORTHRUS_OK;
}

}  // namespace orthrus

extern "C" orthrus_status orthrus_pack(const orthrus_model_cfg *cfg, const orthrus_batch *batch,
                                       orthrus_packed *out, char *err, int32_t err_len) {
  if (err && err_len > 0) err[0] = 0;
  if (!cfg || !batch || !out) return ORTHRUS_EINVAL;
  orthrus::HostPack p;
  orthrus_status st = orthrus::validate_and_pack(*cfg, *batch, p, err, err_len);
  if (st != ORTHRUS_OK) return st;
  if (out->cap_tokens < p.n_tokens || out->cap_items < p.n_items) {
    if (err && err_len > 0) snprintf(err, (size_t)err_len, "output capacity too small");
    return ORTHRUS_ECAPACITY;
  }
  auto put = [](int32_t *dst, const std::vector<int32_t> &v) {
    if (dst && !v.empty()) memcpy(dst, v.data(), v.size() * sizeof(int32_t));
  };
  put(out->cu_q, p.cu_q);
  put(out->pos, p.pos);
  put(out->slot, p.slot);
  put(out->row_item, p.row_item);
  put(out->logit_rows, p.logit_rows);
  put(out->pool_segs, p.pool_segs);
  out->n_embed_rows = p.rows_by_kind[0];
  out->n_prefill_rows = p.rows_by_kind[1];
  out->n_decode_rows = p.rows_by_kind[2];
  out->n_logits = (int32_t)p.logit_rows.size();
  out->n_emb = p.n_emb;
  out->n_pool_segs = (int32_t)(p.pool_segs.size() / 8);
  return ORTHRUS_OK;
}
