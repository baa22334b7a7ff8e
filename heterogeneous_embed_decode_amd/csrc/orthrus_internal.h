// Internal declarations shared by the engine and the kernel launchers.
#pragma once

#include <stdint.h>
#include <vector>

#include "../../include/orthrus.h"

namespace orthrus {

struct HostPack {
  int n_items = 0, n_tokens = 0;
  std::vector<int32_t> cu_q, pos, slot, row_item, logit_rows, pool_segs;
  int rows_by_kind[3] = {0, 0, 0};
  int n_emb = 0;
};

orthrus_status validate_and_pack(const orthrus_model_cfg &cfg, const orthrus_batch &b,
                                 HostPack &p, char *err, int32_t elen);

// ---- attention work list -------------------------------------------------
// One entry per workgroup of the ragged attention launch.
//  CHUNK : rows [q0, q0+qn) of item `item` (local row indices) for KV head
//          `kvh`, against keys [0, ctx + q0 + qn).
//  DECODE: the decode row of `item` for KV head `kvh` against keys
//          [k0, k1); the workgroup writes partial `part`.
enum { WORK_CHUNK = 0, WORK_DECODE = 1 };
// The entry also carries its item's first row, context and page-list
// offset, so a workgroup starts its page and K/V loads from the entry alone
// (one dependent load fewer than reading the item record first).
struct AttnWork {
  int32_t type, item, kvh, q0, qn, k0, k1, part;
  int32_t row0, ctx, page_off, pad;
};
static_assert(sizeof(AttnWork) == 48, "work entries are 12 int32 words");
// Per-item device record used by the attention and combine kernels.
struct DevItem {
  int32_t row0, n, ctx, page_off, kind, part0, n_parts, pad;
};

constexpr int ATTN_ROWS = 128;       // (token, head) rows per chunk workgroup
constexpr int ATTN_WAVES = 4;
constexpr int DEC_SPLIT_VEC = 128;   // keys per decode workgroup, head dims 16 and 32 (32 per wave)
constexpr int DEC_SPLIT_MIN = 128;   // keys per decode workgroup, head dims 64 and 128: 128 ..
constexpr int DEC_SPLIT_MAX = 4096;  // .. 4096, the largest that still gives enough workgroups
constexpr int DEC_MIN_WGS = 2048;    // decode workgroups wanted before a larger split is taken

// keys per decode workgroup the decode path accepts for a head dim
int decode_split_limit(int hd);

// Work list: chunk entries (heaviest first), then decode entries;
// n_chunk counts the former.
void build_attn_work(const orthrus_model_cfg &cfg, const orthrus_batch &b, const HostPack &p,
                     std::vector<AttnWork> &work, std::vector<DevItem> &items, int &n_chunk,
                     int &n_parts);

// ---- static scratch of the allocation-free step (scratch.hip) --------------
// 64 MiB per device: the step metadata at the start (at most
// NOALLOC_META_BYTES), the decode partial results after it.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
constexpr size_t NOALLOC_META_BYTES = size_t(4) << 20;
// Resolve the scratch array's address on `device`, which must be the
// current device; once per device, later calls return at once.  Returns a
// hipError_t value.
int noalloc_scratch_init(int device);
// The resolved address on `device`, or nullptr before noalloc_scratch_init.
void *noalloc_scratch(int device);

// ---- kernel launchers (kernels_*.hip) -------------------------------------
struct LoraArgs {
  const uint16_t *U = nullptr;   // [rows][ldu] bf16, already scaled
  int ldu = 0;
  const uint16_t *Bx = nullptr;  // [N][r] expand matrix
  int r = 0;
  int rows = 0;                  // rows < `rows` get the delta
  int sec1 = 0, sec2 = 0;        // column n in section 0 if n < sec1, 1 if < sec2, else 2
};

enum { EPI_BF16 = 0, EPI_F32 = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_QKV = 4 };

// The one-wave-per-SIMD kernel (kernels_gemm_w4.hip): SwiGLU or plain bf16
// outputs, no adapter, K a multiple of 32, A and B each below 1 GiB, at
// least 256 rows and columns.
bool gemm_w4_eligible(int lda, int ldb, int M, int N, int K, int epi, int b_up_row);
int launch_gemm_w4(const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc, int M, int N, int K,
                   int epi, int b_up_row, float alpha, void *stream);

int launch_gemm(const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc,
                int M, int N, int K, int epi, int b_up_row, float alpha,
                const LoraArgs *lora, void *stream);

// QKV projection with RoPE and the KV append in its epilogue: q (rotated)
// lands in columns [0, Hq*hd) of qkv, k (rotated) and v at each row's KV
// slot, columns [Hq*hd, ldc) of qkv are left unwritten.  Only for the
// shapes qkv_rope_fusable() accepts; the others take launch_gemm followed
// by launch_rope_kv.
struct RopeKv {
  const float *cs = nullptr;      // [M][hd]: cos of the hd/2 angles, then their sin
  const int32_t *slot = nullptr;  // [M] KV slot of each row
  uint16_t *kc = nullptr, *vc = nullptr;
  int n_q_heads = 0, n_kv_heads = 0, page_size = 0;
};
bool qkv_rope_fusable(int M, int Hq, int Hkv, int hd);
int launch_gemm_qkv_rope(const uint16_t *A, int lda, const uint16_t *B, int ldb, uint16_t *qkv, int ldc, int M,
                         int K, const LoraArgs *lora, const RopeKv &rk, void *stream);
// cs[t][i] = cos(pos[t] * inv_freq[i]), cs[t][hd/2 + i] = sin(...), angles in fp64
int launch_rope_table(const int32_t *pos, const double *inv_freq, float *cs, int T, int hd, void *stream);

int launch_embed_rmsnorm(const int32_t *tok, const uint16_t *E, const uint16_t *g, float *x, uint16_t *h,
                         int T, int d, float eps, void *stream);
int launch_rmsnorm(const float *x, const uint16_t *g, uint16_t *h, int T, int d, float eps,
                   void *stream);
int launch_rope_kv(uint16_t *qkv, const int32_t *pos, const int32_t *slot,
                   const double *inv_freq, uint16_t *kc, uint16_t *vc, int T, int Hq, int Hkv,
                   int hd, int ps, void *stream);
// one launch over the work list (chunk entries first, then decode entries)
int launch_attn_ragged(const uint16_t *qkv, int ld_qkv, const uint16_t *kc, const uint16_t *vc,
                       const int32_t *page_ids, const AttnWork *work, int n_work,
                       float *part_ml, float *part_o, uint16_t *o, int ld_o, int Hq, int Hkv, int hd, int ps,
                       void *stream);
int launch_attn_combine(const DevItem *items, const int32_t *dec_items, int n_dec,
                        const float *part_ml, const float *part_o, uint16_t *o, int ld_o,
                        int Hq, int Hkv, int hd, void *stream);
// embedding rows: their 1/rms into rs[row]; logit rows: normalised into hl
int launch_final_norm(const float *x, const uint16_t *g, const int32_t *logit_rows, const int32_t *emb_rows,
                      int n_embed, int n_logit, float *rs, uint16_t *hl, int d, float eps, void *stream);
// fp32 path (kernels_f32.hip)
int launch_gemm_f32(const float *A, int lda, const float *B, int ldb, float *C, int ldc, int M, int N, int K,
                    int epi, int b_up_row, float alpha, const float *U, int ldu, const float *Bx, int r, int lrows,
                    int sec1, int sec2, void *stream);
int launch_rmsnorm_f32(const int32_t *tok, const float *E, float *x, const float *g, float *h, int T, int d,
                       float eps, void *stream);
int launch_final_norm_f32(const float *x, const float *g, const int32_t *logit_rows, int n_embed, int n_logit,
                          float *hf, float *hl, int d, float eps, void *stream);
int launch_rope_kv_f32(float *qkv, const int32_t *pos, const int32_t *slot, const double *inv_freq, float *kc,
                       float *vc, int T, int Hq, int Hkv, int hd, int ps, void *stream);
int launch_attn_f32(const float *qkv, const float *kc, const float *vc, const int32_t *page_ids,
                    const DevItem *items, const int32_t *row_item, const int32_t *pos, float *o, int T, int Hq,
                    int Hkv, int hd, int ps, void *stream);
// compute units of the current device (queried once per process)
int gemm_cu_count();
int launch_gemm_f32_ksplit(const uint16_t *A, int lda, const uint16_t *B, int ldb, float *P, int M, int N, int K,
                           int splits, void *stream);
// U = bf16(scale X A^T).  With a workspace of at least
// lora_shrink_ws_bytes(rows, nr, K) bytes, K is split over several
// workgroups per tile (fp32 partials reduced in a fixed order); with less
// (or none), one workgroup runs a tile's whole K.
size_t lora_shrink_ws_bytes(int rows, int nr, int K);
int launch_lora_shrink(const uint16_t *X, int ldx, const uint16_t *A, int rows, int nr, int K, float scale,
                       uint16_t *U, float *ws, size_t ws_bytes, void *stream);
int launch_sample(const float *logits, int64_t ld, int n_rows, int V, const float *temperature,
                  const float *top_p, const uint32_t *uniforms, int32_t *tokens, void *stream);
int launch_hash_fill(uint16_t *dst, uint64_t n, uint32_t seed, uint32_t tensor_id, uint64_t start, void *stream);
// rs non-null: src is the residual stream and row r pools (src[r] rs[r]) g;
// rs null: src rows are already normalised
int launch_pool(const float *src, const float *rs, const uint16_t *g, const int32_t *segs, int n_segs, float *sum,
                float *wsum, float *kept, float *buf, int buf_rows, float *emb, int d, bool any_l2, void *stream);

}  // namespace orthrus
