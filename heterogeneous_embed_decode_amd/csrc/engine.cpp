// Engine: workspace, metadata staging and the launch sequence of one
// heterogeneous-batch step (forward + emit of the unified runner,
// Efficient Iterative Retrieval with Heterogeneous Batching §3.1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "orthrus_internal.h"

using namespace orthrus;

struct orthrus_engine {
  orthrus_model_cfg cfg{};
  orthrus_weights w{};
  std::vector<orthrus_layer_w> layers;
  uint16_t *kc = nullptr, *vc = nullptr;
  int device = 0;
  // workspace
  float *x = nullptr;
  uint16_t *h = nullptr, *qkv = nullptr, *o = nullptr, *act = nullptr, *U = nullptr;
  float *hf = nullptr;  // fp32 models: the normalised embedding rows
  float *rs = nullptr;  // bf16 models: 1/rms of the embedding rows
  uint16_t *hl = nullptr;
  double *inv_freq = nullptr;
  float *rope_cs = nullptr;  // [T][head_dim] cos/sin table of the step (bf16 models)
  float *lora_ws = nullptr;  // fp32 partial sums of the adapter shrinks
  size_t lora_ws_bytes = 0;
  float *part_ml = nullptr, *part_o = nullptr;
  size_t part_cap = 0;  // in split units
  int32_t *meta_dev = nullptr;
  int32_t *meta_host = nullptr;
  size_t meta_cap = 0;  // int32 words
  hipEvent_t staged{};
  bool staged_pending = false;
  // end of the last step's work, and its stream: a step on another stream
  // waits for it before reusing the workspace and metadata buffers
  hipEvent_t done{};
  hipStream_t last_stream = nullptr;
  bool done_pending = false;
  std::string err;
  // per-layer residual dump (opt-in): [n_layers][dump_cap][d] fp32
  float *dump = nullptr;
  int64_t dump_cap = 0;
  // per-kernel event timing (opt-in)
  bool profiling = false;
  struct Mark {
    const char *name;
    hipEvent_t a, b;
  };
  std::vector<Mark> marks;
  std::vector<hipEvent_t> ev_free;
  // scratch host vectors
  HostPack pack;
  std::vector<AttnWork> work;
  std::vector<DevItem> items;
};

namespace {

// a byte extent the 32-bit buffer offsets of the GEMM kernels can address
// (the buffer resources cover 0x7fffffff bytes)
bool fits_buffer(size_t bytes) { return bytes < 0x7fffffffu; }

orthrus_status hip_fail(orthrus_engine *e, hipError_t r, const char *what) {
  if (e) e->err = std::string(what) + ": " + hipGetErrorString(r);
  return ORTHRUS_EHIP;
}

#define HIPCHK(call, what)                               \
  do {                                                   \
    hipError_t r_ = (call);                              \
    if (r_ != hipSuccess) return hip_fail(eng, r_, what); \
  } while (0)

hipEvent_t take_event(orthrus_engine *e) {
  if (!e->ev_free.empty()) {
    hipEvent_t ev = e->ev_free.back();
    e->ev_free.pop_back();
    return ev;
  }
  hipEvent_t ev{};
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

// Launch `call`; when profiling, bracket it with events on the step stream.
#define LCHK(call, what)                                                  \
  do {                                                                    \
    hipEvent_t ea_ = nullptr, eb_ = nullptr;                              \
    if (eng->profiling) {                                                 \
      ea_ = take_event(eng);                                              \
      eb_ = take_event(eng);                                              \
      if (ea_) (void)hipEventRecord(ea_, s);                              \
    }                                                                     \
    int r_ = (call);                                                      \
    if (r_ != 0) return hip_fail(eng, (hipError_t)r_, what);              \
    if (ea_ && eb_) {                                                     \
      (void)hipEventRecord(eb_, s);                                       \
      eng->marks.push_back({what, ea_, eb_});                             \
    }                                                                     \
  } while (0)

size_t align4(size_t n) { return (n + 3) & ~(size_t)3; }

}  // namespace

namespace orthrus {

void build_attn_work(const orthrus_model_cfg &cfg, const orthrus_batch &b, const HostPack &p,
                     std::vector<AttnWork> &work, std::vector<DevItem> &items, int &n_chunk, int &n_parts) {
  const int G = cfg.n_q_heads / cfg.n_kv_heads;
  const int QB = ATTN_ROWS / G;
  work.clear();
  items.assign(b.n_items, DevItem{});
  // decode split: the largest allowed size that still yields DEC_MIN_WGS
  // workgroups (long splits amortise the per-workgroup merge; short ones
  // fill the chip when there are few decode rows)
  int split = decode_split_limit(cfg.head_dim);
  for (; split > DEC_SPLIT_MIN; split /= 2) {
    long wgs = 0;
    for (int i = 0; i < b.n_items; ++i)
      if (b.items[i].kind == ORTHRUS_DECODE) wgs += (b.items[i].ctx_len + split) / split;
    if (wgs * cfg.n_kv_heads >= DEC_MIN_WGS) break;
  }
  std::vector<AttnWork> dec;
  n_parts = 0;
  for (int i = 0; i < b.n_items; ++i) {
    const orthrus_item &it = b.items[i];
    DevItem &d = items[i];
    d.row0 = p.cu_q[i];
    d.n = it.n_tokens;
    d.ctx = it.ctx_len;
    d.page_off = it.page_off;
    d.kind = it.kind;
    if (it.kind != ORTHRUS_DECODE) {
      for (int g = 0; g < cfg.n_kv_heads; ++g)
        for (int q0 = 0; q0 < it.n_tokens; q0 += QB) {
          const int qn = std::min(QB, it.n_tokens - q0);
          work.push_back({WORK_CHUNK, i, g, q0, qn, 0, it.ctx_len + q0 + qn, 0, d.row0, d.ctx, d.page_off, 0});
        }
    } else {
      const int nk = it.ctx_len + 1;
      const int ns = (nk + split - 1) / split;
      d.part0 = n_parts;
      d.n_parts = ns;
      for (int g = 0; g < cfg.n_kv_heads; ++g)
        for (int s = 0; s < ns; ++s) {
          const int k0 = s * split;
          dec.push_back({WORK_DECODE, i, g, 0, 1, k0, std::min(nk, k0 + split), n_parts + g * ns + s, d.row0, d.ctx,
                         d.page_off, 0});
        }
      n_parts += cfg.n_kv_heads * ns;
    }
  }
  // heaviest chunk tiles first (rows x keys), and longest decode splits
  // first: workgroups start in list order, so the shortest ones fill the
  // last round instead of a long one starting late.  Each entry writes its
  // own partial slot and the combine reads them in a fixed order, so the
  // order changes no result.
  std::stable_sort(work.begin(), work.end(), [](const AttnWork &a, const AttnWork &c) {
    return (long)a.qn * a.k1 > (long)c.qn * c.k1;
  });
  std::stable_sort(dec.begin(), dec.end(),
                   [](const AttnWork &a, const AttnWork &c) { return a.k1 - a.k0 > c.k1 - c.k0; });
  n_chunk = (int)work.size();
  work.insert(work.end(), dec.begin(), dec.end());
}

}  // namespace orthrus

extern "C" {

static std::string g_create_err;  // last failed orthrus_create

const char *orthrus_last_error(const orthrus_engine *eng) { return eng ? eng->err.c_str() : g_create_err.c_str(); }

static void free_all(orthrus_engine *e) {
  for (auto &m : e->marks) {
    (void)hipEventDestroy(m.a);
    (void)hipEventDestroy(m.b);
  }
  e->marks.clear();
  for (auto ev : e->ev_free) (void)hipEventDestroy(ev);
  e->ev_free.clear();
  void *ptrs[] = {e->x, e->h, e->qkv, e->o, e->act, e->U, e->hf, e->rs, e->hl, e->inv_freq,
                  e->rope_cs, e->lora_ws, e->part_ml, e->part_o, e->meta_dev};
  for (void *p : ptrs)
    if (p) (void)hipFree(p);
  if (e->meta_host) (void)hipHostFree(e->meta_host);
  if (e->staged) (void)hipEventDestroy(e->staged);
  if (e->done) (void)hipEventDestroy(e->done);
}

orthrus_status orthrus_create(const orthrus_model_cfg *cfg, const orthrus_weights *w, void *k_pages,
                              void *v_pages, orthrus_engine **out) {
  if (!cfg || !w || !out || !k_pages || !v_pages || !w->layers) return ORTHRUS_EINVAL;
  *out = nullptr;
  const orthrus_model_cfg &c = *cfg;
  const int hd = c.head_dim;
  if (c.n_layers < 1 || c.d_model < 8 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.vocab < 1 ||
      c.ffn_dim < 8 || c.page_size < 1 || c.n_pages < 1 || c.max_tokens < 1 || c.max_items < 1 ||
      c.max_pool_slots < 0 || c.lora_rank < 0)
    return ORTHRUS_EINVAL;
  if (c.dtype != ORTHRUS_BF16 && c.dtype != ORTHRUS_F32) return ORTHRUS_EINVAL;
  if (!(hd == 16 || hd == 32 || hd == 64 || hd == 128)) return ORTHRUS_EINVAL;
  if (c.n_q_heads % c.n_kv_heads) return ORTHRUS_EINVAL;
  const int G = c.n_q_heads / c.n_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return ORTHRUS_EINVAL;
  if (c.d_model % 8 || c.ffn_dim % 8 || c.lora_rank % 8 || c.d_model > 8192 || c.lora_rank > 64)
    return ORTHRUS_EINVAL;
  {
    // GEMM operands and the fp32 residual are addressed through 32-bit
    // buffer offsets: every row-major operand of a step must stay below 2 GiB
    const size_t qkv_w = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * hd;
    const size_t widest = std::max({(size_t)c.d_model, qkv_w, (size_t)c.ffn_dim});
    if (!fits_buffer((size_t)c.max_tokens * widest * 4) || !fits_buffer((size_t)c.vocab * c.d_model * 2) ||
        !fits_buffer((size_t)2 * c.ffn_dim * c.d_model * 2) || !fits_buffer(qkv_w * c.d_model * 2))
      return ORTHRUS_EINVAL;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const orthrus_layer_w &L = w->layers[l];
    if (!L.w_qkv || !L.w_o || !L.w_gate_up || !L.w_down || !L.g_attn || !L.g_ffn) return ORTHRUS_EINVAL;
    if (c.lora_rank > 0 && (!L.lora_a_qkv || !L.lora_b_qkv || !L.lora_a_o || !L.lora_b_o))
      return ORTHRUS_EINVAL;
  }
  if (!w->tok_emb || !w->lm_head || !w->g_final) return ORTHRUS_EINVAL;

  orthrus_engine *eng = new orthrus_engine();
  eng->cfg = c;
  eng->w = *w;
  eng->layers.assign(w->layers, w->layers + c.n_layers);
  eng->w.layers = eng->layers.data();
  eng->kc = (uint16_t *)k_pages;
  eng->vc = (uint16_t *)v_pages;
  auto bail = [&](orthrus_status s, const char *what, hipError_t r) {
    g_create_err = std::string(what) + ": " + hipGetErrorString(r);
    free_all(eng);
    delete eng;
    return s;
  };
  hipError_t r = hipGetDevice(&eng->device);
  if (r != hipSuccess) return bail(ORTHRUS_EHIP, "hipGetDevice", r);
  // the allocation-free step's static scratch: its address on this device
  if ((r = (hipError_t)noalloc_scratch_init(eng->device)) != hipSuccess)
    return bail(ORTHRUS_EHIP, "hipGetSymbolAddress(scratch)", r);
  const size_t T = c.max_tokens, d = c.d_model;
  const size_t qkvd = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * hd, qd = (size_t)c.n_q_heads * hd;
  const size_t es = c.dtype == ORTHRUS_F32 ? 4 : 2;  // bytes of an activation element
  struct {
    void **p;
    size_t bytes;
  } allocs[] = {
      {(void **)&eng->x, T * d * 4},
      {(void **)&eng->h, T * std::max(d, qd) * es},
      {(void **)&eng->qkv, T * qkvd * es},
      {(void **)&eng->o, T * qd * es},
      {(void **)&eng->act, T * (size_t)c.ffn_dim * es},
      {(void **)&eng->U, T * (size_t)std::max(3 * c.lora_rank, 8) * es},
      {(void **)&eng->hf, c.dtype == ORTHRUS_F32 ? T * d * 4 : 4},
      {(void **)&eng->rs, T * 4},
      {(void **)&eng->hl, T * d * es},
      {(void **)&eng->inv_freq, (size_t)hd / 2 * 8},
      {(void **)&eng->rope_cs, T * hd * 4},
  };
  for (auto &a : allocs)
    if ((r = hipMalloc(a.p, a.bytes)) != hipSuccess) return bail(ORTHRUS_ENOMEM, "hipMalloc", r);
  if (c.lora_rank > 0 && c.dtype != ORTHRUS_F32) {
    // the shrinks' split-K partial sums: the most that the QKV (3r columns
    // over d) or O (r columns over Hq*hd) shrink needs at up to max_tokens
    // embedding rows (fewer rows take more splits; within a 64-row tile row
    // the need grows with the rows)
    for (size_t rows = 64;; rows += 64) {
      const int rr = (int)std::min(rows, T);
      eng->lora_ws_bytes = std::max({eng->lora_ws_bytes, lora_shrink_ws_bytes(rr, 3 * c.lora_rank, (int)d),
                                     lora_shrink_ws_bytes(rr, c.lora_rank, (int)qd)});
      if ((size_t)rr == T) break;
    }
    if (eng->lora_ws_bytes && (r = hipMalloc(&eng->lora_ws, eng->lora_ws_bytes)) != hipSuccess)
      return bail(ORTHRUS_ENOMEM, "hipMalloc", r);
  }
  std::vector<double> inv(hd / 2);
  for (int i = 0; i < hd / 2; ++i) inv[i] = std::pow((double)c.rope_theta, -2.0 * i / hd);
  if ((r = hipMemcpy(eng->inv_freq, inv.data(), inv.size() * 8, hipMemcpyHostToDevice)) != hipSuccess)
    return bail(ORTHRUS_EHIP, "hipMemcpy", r);
  // metadata staging, pinned host and device, sized for the allocation-free
  // step's largest metadata block; orthrus_step grows both when a batch needs more
  eng->meta_cap = NOALLOC_META_BYTES / 4;
  if ((r = hipMalloc(&eng->meta_dev, eng->meta_cap * 4)) != hipSuccess)
    return bail(ORTHRUS_ENOMEM, "hipMalloc", r);
  if ((r = hipHostMalloc(&eng->meta_host, eng->meta_cap * 4, hipHostMallocDefault)) != hipSuccess)
    return bail(ORTHRUS_ENOMEM, "hipHostMalloc", r);
  if ((r = hipEventCreateWithFlags(&eng->staged, hipEventDisableTiming)) != hipSuccess ||
      (r = hipEventCreateWithFlags(&eng->done, hipEventDisableTiming)) != hipSuccess)
    return bail(ORTHRUS_EHIP, "hipEventCreate", r);
  g_create_err.clear();
  *out = eng;
  return ORTHRUS_OK;
}

void orthrus_destroy(orthrus_engine *eng) {
  if (!eng) return;
  (void)hipSetDevice(eng->device);
  (void)hipDeviceSynchronize();
  free_all(eng);
  delete eng;
}

static orthrus_status step_impl(orthrus_engine *eng, const orthrus_batch *batch, const orthrus_pool_state *pool,
                                float *logits, int32_t logits_cap_rows, float *emb, int32_t emb_cap_rows,
                                int32_t *n_logits, int32_t *n_emb, int32_t *logit_req_ids, int32_t *emb_req_ids,
                                float *hidden_out, void *stream, bool noalloc) {
  if (!eng) return ORTHRUS_EINVAL;
  eng->err.clear();
  if (!batch || !pool) {
    eng->err = "null batch or pool state";
    return ORTHRUS_EINVAL;
  }
  const orthrus_model_cfg &c = eng->cfg;
  char msg[256];
  HostPack &p = eng->pack;
  orthrus_status st = validate_and_pack(c, *batch, p, msg, sizeof msg);
  if (st != ORTHRUS_OK) {
    eng->err = msg;
    return st;
  }
  const int G = (int)p.logit_rows.size();
  if (G > logits_cap_rows || p.n_emb > emb_cap_rows) {
    eng->err = "output capacity too small";
    return ORTHRUS_ECAPACITY;
  }
  if ((G > 0 && !logits) || (p.n_emb > 0 && !emb) ||
      (p.rows_by_kind[0] > 0 && (!pool->sum || !pool->wsum || !pool->kept))) {
    eng->err = "null output or pool buffer";
    return ORTHRUS_EINVAL;
  }
  for (size_t k = 0; k < p.pool_segs.size(); k += 8)
    if ((p.pool_segs[k + 3] & ~ORTHRUS_POOL_L2) == ORTHRUS_POOL_BUFFER &&
        (!pool->buf || p.pool_segs[k + 6] + p.pool_segs[k + 1] > pool->buf_rows)) {
      eng->err = "pooling buffer missing or too short for a BUFFER item";
      return ORTHRUS_ECAPACITY;
    }
  if (n_logits) *n_logits = G;
  if (n_emb) *n_emb = p.n_emb;
  if (logit_req_ids)
    for (int k = 0; k < G; ++k) logit_req_ids[k] = batch->items[p.row_item[p.logit_rows[k]]].req_id;
  if (emb_req_ids) {
    int k = 0;
    for (int i = 0; i < batch->n_items; ++i)
      if (batch->items[i].kind == ORTHRUS_EMBED && batch->items[i].is_last) emb_req_ids[k++] = batch->items[i].req_id;
  }
  const int T = p.n_tokens;
  if (eng->dump && T > eng->dump_cap) {
    eng->err = "batch has more rows than the layer dump holds";
    return ORTHRUS_ECAPACITY;
  }
  if (T == 0) return ORTHRUS_OK;

  int n_parts = 0, n_chunk = 0;
  build_attn_work(c, *batch, p, eng->work, eng->items, n_chunk, n_parts);
  const int n_dec_work = (int)eng->work.size() - n_chunk;
  std::vector<int32_t> dec_items;
  bool multi_split = false;  // some decode row needs the combine kernel
  for (int i = 0; i < batch->n_items; ++i)
    if (batch->items[i].kind == ORTHRUS_DECODE) {
      dec_items.push_back(i);
      multi_split |= eng->items[i].n_parts > 1;
    }

  HIPCHK(hipSetDevice(eng->device), "hipSetDevice");
  hipStream_t s = (hipStream_t)stream;

  // embedding rows the pooling heads read from the final norm: every row
  // of a mean, weighted-mean or buffered segment, the first row of a CLS
  // segment that starts its request, the last row of a LAST segment
  // (norm_subset false: all embedding rows, in order)
  const size_t n_segs = p.pool_segs.size() / 8;
  std::vector<int32_t> norm_rows;
  bool norm_subset = false;
  {
    size_t need = 0;
    for (size_t q = 0; q < n_segs; ++q) {
      const int32_t *sg = &p.pool_segs[q * 8];
      const int kind = sg[3] & ~ORTHRUS_POOL_L2;
      if (kind == ORTHRUS_POOL_CLS) need += sg[4] ? 1 : 0;
      else if (kind == ORTHRUS_POOL_LAST) need += 1;
      else need += sg[1];
    }
    if (need < (size_t)p.rows_by_kind[0]) {
      norm_subset = true;
      norm_rows.reserve(need);
      for (size_t q = 0; q < n_segs; ++q) {
        const int32_t *sg = &p.pool_segs[q * 8];
        const int kind = sg[3] & ~ORTHRUS_POOL_L2;
        if (kind == ORTHRUS_POOL_CLS) {
          if (sg[4]) norm_rows.push_back(sg[0]);
        } else if (kind == ORTHRUS_POOL_LAST) {
          norm_rows.push_back(sg[0] + sg[1] - 1);
        } else {
          for (int r = 0; r < sg[1]; ++r) norm_rows.push_back(sg[0] + r);
        }
      }
    }
  }

  // metadata block (int32 words, 16-byte aligned sections)
  size_t off = 0;
  const size_t o_tok = off; off = align4(off + T);
  const size_t o_pos = off; off = align4(off + T);
  const size_t o_slot = off; off = align4(off + T);
  const size_t o_pages = off; off = align4(off + (size_t)batch->n_page_ids);
  const size_t o_logit = off; off = align4(off + G);
  const size_t o_segs = off; off = align4(off + n_segs * 8);
  const size_t o_dec = off; off = align4(off + dec_items.size());
  const size_t o_items = off; off = align4(off + eng->items.size() * 8);
  const size_t o_work = off; off = align4(off + eng->work.size() * (sizeof(AttnWork) / 4));
  const size_t o_norm = off; off = align4(off + norm_rows.size());
  const size_t o_ritem = off; off = align4(off + (c.dtype == ORTHRUS_F32 ? (size_t)T : 0));
  const size_t words = std::max<size_t>(off, 4);
  const int Gq = c.n_q_heads / c.n_kv_heads;
  int32_t *meta_dev = eng->meta_dev;
  float *part_ml = eng->part_ml, *part_o = eng->part_o;
  if (noalloc) {
    // metadata and decode partials in the static scratch: refuse what does
    // not fit before any device work
    char *base = (char *)noalloc_scratch(eng->device);
    const size_t ml_bytes = ((size_t)n_parts * Gq * 2 * 4 + 255) & ~(size_t)255;
    const size_t o_bytes = (size_t)n_parts * Gq * c.head_dim * 4;
    if (!base) {
      eng->err = "static scratch not resolved on this device";
      return ORTHRUS_EHIP;
    }
    if (words * 4 > NOALLOC_META_BYTES || words > eng->meta_cap) {
      eng->err = "step metadata exceeds the allocation-free limit (" + std::to_string(NOALLOC_META_BYTES / 4) +
                 " int32 words)";
      return ORTHRUS_ECAPACITY;
    }
    if (ml_bytes + o_bytes > NOALLOC_SCRATCH_BYTES - NOALLOC_META_BYTES) {
      eng->err = "decode partial results exceed the allocation-free scratch (" +
                 std::to_string((NOALLOC_SCRATCH_BYTES - NOALLOC_META_BYTES) >> 20) + " MiB)";
      return ORTHRUS_ECAPACITY;
    }
    meta_dev = (int32_t *)base;
    part_ml = (float *)(base + NOALLOC_META_BYTES);
    part_o = (float *)(base + NOALLOC_META_BYTES + ml_bytes);
  }
  if (eng->staged_pending) {
    HIPCHK(hipEventSynchronize(eng->staged), "hipEventSynchronize");
    eng->staged_pending = false;
  }
  if (!noalloc && words > eng->meta_cap) {
    const size_t cap = words * 2;
    if (eng->meta_dev) {
      HIPCHK(hipDeviceSynchronize(), "hipDeviceSynchronize");
      (void)hipFree(eng->meta_dev);
      (void)hipHostFree(eng->meta_host);
      eng->meta_dev = nullptr;
      eng->meta_host = nullptr;
      eng->meta_cap = 0;
    }
    if (hipMalloc(&eng->meta_dev, cap * 4) != hipSuccess ||
        hipHostMalloc(&eng->meta_host, cap * 4, hipHostMallocDefault) != hipSuccess) {
      eng->err = "metadata allocation failed";
      return ORTHRUS_ENOMEM;
    }
    eng->meta_cap = cap;
    meta_dev = eng->meta_dev;
  }
  if (!noalloc && (size_t)n_parts > eng->part_cap) {
    const size_t cap = (size_t)n_parts * 2;
    HIPCHK(hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (eng->part_ml) (void)hipFree(eng->part_ml);
    if (eng->part_o) (void)hipFree(eng->part_o);
    eng->part_ml = eng->part_o = nullptr;
    eng->part_cap = 0;
    if (hipMalloc(&eng->part_ml, cap * Gq * 2 * 4) != hipSuccess ||
        hipMalloc(&eng->part_o, cap * Gq * (size_t)c.head_dim * 4) != hipSuccess) {
      eng->err = "partial buffer allocation failed";
      return ORTHRUS_ENOMEM;
    }
    eng->part_cap = cap;
    part_ml = eng->part_ml;
    part_o = eng->part_o;
  }
  int32_t *mh = eng->meta_host;
  memcpy(mh + o_tok, batch->token_ids, (size_t)T * 4);
  memcpy(mh + o_pos, p.pos.data(), (size_t)T * 4);
  memcpy(mh + o_slot, p.slot.data(), (size_t)T * 4);
  if (batch->n_page_ids) memcpy(mh + o_pages, batch->page_ids, (size_t)batch->n_page_ids * 4);
  if (G) memcpy(mh + o_logit, p.logit_rows.data(), (size_t)G * 4);
  if (n_segs) memcpy(mh + o_segs, p.pool_segs.data(), n_segs * 8 * 4);
  if (!dec_items.empty()) memcpy(mh + o_dec, dec_items.data(), dec_items.size() * 4);
  if (!eng->items.empty()) memcpy(mh + o_items, eng->items.data(), eng->items.size() * 32);
  if (!eng->work.empty()) memcpy(mh + o_work, eng->work.data(), eng->work.size() * sizeof(AttnWork));
  if (!norm_rows.empty()) memcpy(mh + o_norm, norm_rows.data(), norm_rows.size() * 4);
  if (c.dtype == ORTHRUS_F32) memcpy(mh + o_ritem, p.row_item.data(), (size_t)T * 4);
  if (eng->done_pending && eng->last_stream != s)
    HIPCHK(hipStreamWaitEvent(s, eng->done, 0), "hipStreamWaitEvent");
  HIPCHK(hipMemcpyAsync(meta_dev, mh, words * 4, hipMemcpyHostToDevice, s), "metadata upload");
  HIPCHK(hipEventRecord(eng->staged, s), "hipEventRecord");
  eng->staged_pending = true;

  const int32_t *d_tok = meta_dev + o_tok, *d_pos = meta_dev + o_pos;
  const int32_t *d_slot = meta_dev + o_slot, *d_pages = meta_dev + o_pages;
  const int32_t *d_logit = meta_dev + o_logit, *d_segs = meta_dev + o_segs;
  const int32_t *d_dec = meta_dev + o_dec;
  const DevItem *d_items = (const DevItem *)(meta_dev + o_items);
  const AttnWork *d_work = (const AttnWork *)(meta_dev + o_work);

  const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, F = c.ffn_dim;
  const int qd = Hq * hd, kvd = Hkv * hd, qkvd = qd + 2 * kvd, r = c.lora_rank;
  const int TE = p.rows_by_kind[0];
  const size_t layer_kv = (size_t)c.n_pages * Hkv * c.page_size * hd;

  if (c.dtype == ORTHRUS_F32) {
    // fp32 path: the same forward on fp32 weights, pages and activations
    float *h = (float *)eng->h, *qkv = (float *)eng->qkv, *o = (float *)eng->o, *act = (float *)eng->act;
    float *U = (float *)eng->U, *hl = (float *)eng->hl;
    const int32_t *d_ritem = meta_dev + o_ritem;
    for (int l = 0; l < c.n_layers; ++l) {
      const orthrus_layer_w &L = eng->layers[l];
      float *kc = (float *)eng->kc + (size_t)l * layer_kv, *vc = (float *)eng->vc + (size_t)l * layer_kv;
      const bool lora = r > 0 && TE > 0;
      LCHK(launch_rmsnorm_f32(l == 0 ? d_tok : nullptr, (const float *)eng->w.tok_emb, eng->x,
                              (const float *)L.g_attn, h, T, d, c.rms_eps, s),
           "rmsnorm_f32");
      if (lora)
        LCHK(launch_gemm_f32(h, d, (const float *)L.lora_a_qkv, d, U, 3 * r, TE, 3 * r, d, EPI_F32, 0,
                             c.lora_scale, nullptr, 0, nullptr, 0, 0, 0, 0, s),
             "lora_shrink_qkv_f32");
      LCHK(launch_gemm_f32(h, d, (const float *)L.w_qkv, d, qkv, qkvd, T, qkvd, d, EPI_F32, 0, 1.f,
                           lora ? U : nullptr, 3 * r, (const float *)L.lora_b_qkv, r, TE, qd, qd + kvd, s),
           "gemm_qkv_f32");
      LCHK(launch_rope_kv_f32(qkv, d_pos, d_slot, eng->inv_freq, kc, vc, T, Hq, Hkv, hd, c.page_size, s),
           "rope_kv_f32");
      LCHK(launch_attn_f32(qkv, kc, vc, d_pages, d_items, d_ritem, d_pos, o, T, Hq, Hkv, hd, c.page_size, s),
           "attn_f32");
      if (lora)
        LCHK(launch_gemm_f32(o, qd, (const float *)L.lora_a_o, qd, U, r, TE, r, qd, EPI_F32, 0, c.lora_scale,
                             nullptr, 0, nullptr, 0, 0, 0, 0, s),
             "lora_shrink_o_f32");
      LCHK(launch_gemm_f32(o, qd, (const float *)L.w_o, qd, eng->x, d, T, d, qd, EPI_RESID, 0, 1.f,
                           lora ? U : nullptr, r, (const float *)L.lora_b_o, r, TE, d, d, s),
           "gemm_o_f32");
      LCHK(launch_rmsnorm_f32(nullptr, nullptr, eng->x, (const float *)L.g_ffn, h, T, d, c.rms_eps, s),
           "rmsnorm_f32");
      LCHK(launch_gemm_f32(h, d, (const float *)L.w_gate_up, d, act, F, T, F, d, EPI_SWIGLU, F, 1.f, nullptr, 0,
                           nullptr, 0, 0, 0, 0, s),
           "gemm_gate_up_f32");
      LCHK(launch_gemm_f32(act, F, (const float *)L.w_down, F, eng->x, d, T, d, F, EPI_RESID, 0, 1.f, nullptr,
                           0, nullptr, 0, 0, 0, 0, s),
           "gemm_down_f32");
      if (eng->dump)
        HIPCHK(hipMemcpyAsync(eng->dump + (size_t)l * eng->dump_cap * d, eng->x, (size_t)T * d * 4,
                              hipMemcpyDeviceToDevice, s),
               "layer dump copy");
    }
    if (hidden_out)
      HIPCHK(hipMemcpyAsync(hidden_out, eng->x, (size_t)T * d * 4, hipMemcpyDeviceToDevice, s), "hidden copy");
    LCHK(launch_final_norm_f32(eng->x, (const float *)eng->w.g_final, d_logit, TE, G, eng->hf, hl, d, c.rms_eps,
                               s),
         "final_norm_f32");
    if (G > 0)
      LCHK(launch_gemm_f32(hl, d, (const float *)eng->w.lm_head, d, logits, c.vocab, G, c.vocab, d, EPI_F32, 0,
                           1.f, nullptr, 0, nullptr, 0, 0, 0, 0, s),
           "lm_head_f32");
  } else {
  // RoPE and the KV append run in the QKV projection's epilogue where its
  // shape allows, from one cos/sin table per step
  const bool fuse_rope = qkv_rope_fusable(T, Hq, Hkv, hd);
  RopeKv rk{};
  if (fuse_rope) {
    LCHK(launch_rope_table(d_pos, eng->inv_freq, eng->rope_cs, T, hd, s), "rope_table");
    rk.cs = eng->rope_cs; rk.slot = d_slot;
    rk.n_q_heads = Hq; rk.n_kv_heads = Hkv; rk.page_size = c.page_size;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const orthrus_layer_w &L = eng->layers[l];
    uint16_t *kc = eng->kc + (size_t)l * layer_kv, *vc = eng->vc + (size_t)l * layer_kv;
    const bool lora = r > 0 && TE > 0;
    if (l == 0)
      LCHK(launch_embed_rmsnorm(d_tok, (const uint16_t *)eng->w.tok_emb, (const uint16_t *)L.g_attn, eng->x,
                                eng->h, T, d, c.rms_eps, s),
           "embed_rmsnorm");
    else
      LCHK(launch_rmsnorm(eng->x, (const uint16_t *)L.g_attn, eng->h, T, d, c.rms_eps, s), "rmsnorm");
    LoraArgs la{};
    if (lora) {
      LCHK(launch_lora_shrink(eng->h, d, (const uint16_t *)L.lora_a_qkv, TE, 3 * r, d, c.lora_scale, eng->U,
                              eng->lora_ws, eng->lora_ws_bytes, s),
           "lora_shrink_qkv");
      la.U = eng->U; la.ldu = 3 * r; la.Bx = (const uint16_t *)L.lora_b_qkv; la.r = r; la.rows = TE;
      la.sec1 = qd; la.sec2 = qd + kvd;
    }
    if (fuse_rope) {
      rk.kc = kc; rk.vc = vc;
      LCHK(launch_gemm_qkv_rope(eng->h, d, (const uint16_t *)L.w_qkv, d, eng->qkv, qkvd, T, d,
                                lora ? &la : nullptr, rk, s),
           "gemm_qkv_rope");
    } else {
      LCHK(launch_gemm(eng->h, d, (const uint16_t *)L.w_qkv, d, eng->qkv, qkvd, T, qkvd, d, EPI_BF16, 0, 1.f,
                       lora ? &la : nullptr, s),
           "gemm_qkv");
      LCHK(launch_rope_kv(eng->qkv, d_pos, d_slot, eng->inv_freq, kc, vc, T, Hq, Hkv, hd, c.page_size, s),
           "rope_kv");
    }
    LCHK(launch_attn_ragged(eng->qkv, qkvd, kc, vc, d_pages, d_work, n_chunk + n_dec_work, part_ml,
                            part_o, eng->o, qd, Hq, Hkv, hd, c.page_size, s),
         "attn_ragged");
    if (multi_split)
      LCHK(launch_attn_combine(d_items, d_dec, (int)dec_items.size(), part_ml, part_o, eng->o, qd,
                               Hq, Hkv, hd, s),
           "attn_combine");
    if (lora) {
      LCHK(launch_lora_shrink(eng->o, qd, (const uint16_t *)L.lora_a_o, TE, r, qd, c.lora_scale, eng->U,
                              eng->lora_ws, eng->lora_ws_bytes, s),
           "lora_shrink_o");
      la.ldu = r; la.Bx = (const uint16_t *)L.lora_b_o; la.sec1 = d; la.sec2 = d;
    }
    LCHK(launch_gemm(eng->o, qd, (const uint16_t *)L.w_o, qd, eng->x, d, T, d, qd, EPI_RESID, 0, 1.f,
                     lora ? &la : nullptr, s),
         "gemm_o");
    LCHK(launch_rmsnorm(eng->x, (const uint16_t *)L.g_ffn, eng->h, T, d, c.rms_eps, s), "rmsnorm");
    LCHK(launch_gemm(eng->h, d, (const uint16_t *)L.w_gate_up, d, eng->act, F, T, F, d, EPI_SWIGLU, F, 1.f,
                     nullptr, s),
         "gemm_gate_up");
    LCHK(launch_gemm(eng->act, F, (const uint16_t *)L.w_down, F, eng->x, d, T, d, F, EPI_RESID, 0, 1.f,
                     nullptr, s),
         "gemm_down");
    if (eng->dump)
      HIPCHK(hipMemcpyAsync(eng->dump + (size_t)l * eng->dump_cap * d, eng->x, (size_t)T * d * 4,
                            hipMemcpyDeviceToDevice, s),
             "layer dump copy");
  }
  if (hidden_out)
    HIPCHK(hipMemcpyAsync(hidden_out, eng->x, (size_t)T * d * 4, hipMemcpyDeviceToDevice, s), "hidden copy");
  LCHK(launch_final_norm(eng->x, (const uint16_t *)eng->w.g_final, d_logit,
                         norm_subset ? meta_dev + o_norm : nullptr,
                         norm_subset ? (int)norm_rows.size() : TE, G, eng->rs, eng->hl, d, c.rms_eps, s),
       "final_norm");
  if (G > 0)
    LCHK(launch_gemm(eng->hl, d, (const uint16_t *)eng->w.lm_head, d, logits, c.vocab, G, c.vocab, d, EPI_F32,
                     0, 1.f, nullptr, s),
         "lm_head");
  }
  if (n_segs) {
    bool any_l2 = false;  // an emitted embedding is scaled to unit length
    for (size_t q = 0; q < n_segs; ++q) any_l2 |= (p.pool_segs[q * 8 + 3] & ORTHRUS_POOL_L2) && p.pool_segs[q * 8 + 5];
    // bf16 models pool the residual rows through the final norm's 1/rms;
    // fp32 models pool the rows their final norm wrote
    const bool f32 = c.dtype == ORTHRUS_F32;
    LCHK(launch_pool(f32 ? eng->hf : eng->x, f32 ? nullptr : eng->rs, (const uint16_t *)eng->w.g_final, d_segs,
                     (int)n_segs, pool->sum, pool->wsum, pool->kept, pool->buf, pool->buf_rows, emb, d, any_l2, s),
         "pool");
  }
  HIPCHK(hipEventRecord(eng->done, s), "hipEventRecord");
  eng->last_stream = s;
  eng->done_pending = true;
  return ORTHRUS_OK;
}

orthrus_status orthrus_step(orthrus_engine *eng, const orthrus_batch *batch, const orthrus_pool_state *pool,
                            float *logits, int32_t logits_cap_rows, float *emb, int32_t emb_cap_rows,
                            int32_t *n_logits, int32_t *n_emb, int32_t *logit_req_ids, int32_t *emb_req_ids,
                            float *hidden_out, void *stream) {
  return step_impl(eng, batch, pool, logits, logits_cap_rows, emb, emb_cap_rows, n_logits, n_emb, logit_req_ids,
                   emb_req_ids, hidden_out, stream, false);
}

orthrus_status orthrus_step_noalloc(orthrus_engine *eng, const orthrus_batch *batch, const orthrus_pool_state *pool,
                                    float *logits, int32_t logits_cap_rows, float *emb, int32_t emb_cap_rows,
                                    int32_t *n_logits, int32_t *n_emb, int32_t *logit_req_ids,
                                    int32_t *emb_req_ids, float *hidden_out, void *stream) {
  return step_impl(eng, batch, pool, logits, logits_cap_rows, emb, emb_cap_rows, n_logits, n_emb, logit_req_ids,
                   emb_req_ids, hidden_out, stream, true);
}

orthrus_status orthrus_set_layer_dump(orthrus_engine *eng, float *dst, int64_t cap_rows) {
  if (!eng || (dst && cap_rows < 1)) return ORTHRUS_EINVAL;
  eng->dump = dst;
  eng->dump_cap = dst ? cap_rows : 0;
  return ORTHRUS_OK;
}

orthrus_status orthrus_profile(orthrus_engine *eng, int32_t enable) {
  if (!eng) return ORTHRUS_EINVAL;
  eng->profiling = enable != 0;
  return ORTHRUS_OK;
}

int32_t orthrus_profile_read(orthrus_engine *eng, char *json, int32_t len) {
  if (!eng) return -1;
  struct Acc {
    std::string name;
    int count = 0;
    double ms = 0, min_ms = 1e30, max_ms = 0;
  };
  std::vector<Acc> acc;
  const bool consume = json != nullptr && len > 0;
  for (auto &m : eng->marks) {
    float ms = 0.f;
    if (hipEventSynchronize(m.b) != hipSuccess || hipEventElapsedTime(&ms, m.a, m.b) != hipSuccess) ms = -1.f;
    if (consume) {
      eng->ev_free.push_back(m.a);
      eng->ev_free.push_back(m.b);
    }
    Acc *a = nullptr;
    for (auto &x : acc)
      if (x.name == m.name) a = &x;
    if (!a) {
      acc.push_back(Acc{m.name});
      a = &acc.back();
    }
    a->count++;
    a->ms += ms;
    a->min_ms = std::min(a->min_ms, (double)ms);
    a->max_ms = std::max(a->max_ms, (double)ms);
  }
  if (consume) eng->marks.clear();
  std::string out = "{";
  for (size_t i = 0; i < acc.size(); ++i) {
    char buf[256];
    snprintf(buf, sizeof buf, "%s\"%s\": {\"count\": %d, \"total_ms\": %.6f, \"min_ms\": %.6f, \"max_ms\": %.6f}",
             i ? ", " : "", acc[i].name.c_str(), acc[i].count, acc[i].ms, acc[i].min_ms, acc[i].max_ms);
    out += buf;
  }
  out += "}";
  if (json && len > 0) {
    const size_t n = std::min(out.size(), (size_t)len - 1);
    memcpy(json, out.data(), n);
    json[n] = 0;
  }
  return (int32_t)out.size();
}

orthrus_status orthrus_fill_hash_bf16(void *dst, uint64_t n, uint32_t seed, uint32_t tensor_id, uint64_t start,
                                     void *stream) {
  if (!dst && n) return ORTHRUS_EINVAL;
  return launch_hash_fill((uint16_t *)dst, n, seed, tensor_id, start, stream) ? ORTHRUS_EHIP : ORTHRUS_OK;
}

orthrus_status orthrus_gemm_bf16(const void *A, int32_t lda, const void *B, int32_t ldb, void *C, int32_t ldc,
                                 int32_t M, int32_t N, int32_t K, int32_t epilogue, int32_t b_up_row,
                                 void *stream) {
  if (!A || !B || !C || M < 0 || N < 0 || K < 8 || K % 8 || lda % 8 || ldb % 8 || lda < K || ldb < K ||
      epilogue < 0 || epilogue > 3 || ldc < N)
    return ORTHRUS_EINVAL;
  if (epilogue == EPI_SWIGLU && b_up_row < N) return ORTHRUS_EINVAL;
  // the kernels address A, B and a residual C through 32-bit buffer offsets
  if (M > 0 && N > 0) {
    const size_t b_rows = epilogue == EPI_SWIGLU ? (size_t)b_up_row + N : (size_t)N;
    if (!fits_buffer(((size_t)(M - 1) * lda + K) * 2) || !fits_buffer(((b_rows - 1) * ldb + K) * 2) ||
        (epilogue == EPI_RESID && !fits_buffer(((size_t)(M - 1) * ldc + N) * 4)))
      return ORTHRUS_EINVAL;
  }
  const int r = launch_gemm((const uint16_t *)A, lda, (const uint16_t *)B, ldb, C, ldc, M, N, K, epilogue,
                            b_up_row, 1.f, nullptr, stream);
  return r ? ORTHRUS_EHIP : ORTHRUS_OK;
}

orthrus_status orthrus_lora_shrink_bf16(const void *X, int32_t ldx, const void *A, int32_t rows, int32_t nr,
                                        int32_t K, float scale, void *U, void *workspace, int64_t workspace_bytes,
                                        void *stream) {
  if (rows < 0 || nr < 0 || K < 8 || K % 8 || ldx < K || ldx % 8 || workspace_bytes < 0) return ORTHRUS_EINVAL;
  if (rows == 0 || nr == 0) return ORTHRUS_OK;
  if (!X || !A || !U) return ORTHRUS_EINVAL;
  if (!fits_buffer(((size_t)(rows - 1) * ldx + K) * 2) || !fits_buffer((size_t)nr * K * 2)) return ORTHRUS_EINVAL;
  return launch_lora_shrink((const uint16_t *)X, ldx, (const uint16_t *)A, rows, nr, K, scale, (uint16_t *)U,
                            (float *)workspace, workspace ? (size_t)workspace_bytes : 0, stream)
             ? ORTHRUS_EHIP
             : ORTHRUS_OK;
}

orthrus_status orthrus_sample(const float *logits, int64_t ld, int32_t n_rows, int32_t vocab,
                              const float *temperature, const float *top_p, const uint32_t *uniforms,
                              int32_t *tokens, void *stream) {
  if (n_rows < 0 || vocab < 1 || ld < vocab) return ORTHRUS_EINVAL;
  if (n_rows == 0) return ORTHRUS_OK;
  if (!logits || !tokens || (temperature && !uniforms)) return ORTHRUS_EINVAL;
  return launch_sample(logits, ld, n_rows, vocab, temperature, top_p, uniforms, tokens, stream) ? ORTHRUS_EHIP
                                                                                                : ORTHRUS_OK;
}

}  // extern "C"
