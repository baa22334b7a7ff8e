// Memory-bound kernels of the step: token-embedding gather, RMSNorm,
// RoPE + paged KV append, final norm with the row split between LM head
// and pooler, and the segmented incremental pooling update.
//
// Efficient Iterative Retrieval with Heterogeneous Batching: §3.1 (one
// shared forward for every item type), §2.2 Generation (each processed
// token appends its KV entries), §3.2 Batch Unit (output stages work on
// contiguous, type-sorted row slices), §3.3 Incremental Pooler with the
// agihunt summary (running weighted sum and weight total, then divide; CLS
// and last-token heads keep the chosen hidden state).
#include "device_common.h"
#include "orthrus_internal.h"

#include <algorithm>

namespace orthrus {

__device__ __forceinline__ float block_sum_256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Rows of up to NORM_MAXV * 1024 values are held in registers (float4 per
// thread and slot) between the sum of squares and the scaled write-out, so
// x is read from HBM once.
constexpr int NORM_MAXV = 8;

__device__ __forceinline__ void norm_write_bf16(const float4 *v, const uint16_t *g, uint16_t *hr, int nv4,
                                                float inv) {
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c >= nv4) break;
    const uint2 gw = *(const uint2 *)(g + c * 4);
    uint2 o;
    o.x = pack_bf2(v[j].x * inv * lo_bf(gw.x), v[j].y * inv * hi_bf(gw.x));
    o.y = pack_bf2(v[j].z * inv * lo_bf(gw.y), v[j].w * inv * hi_bf(gw.y));
    *(uint2 *)(hr + c * 4) = o;
  }
}

// x[t] = fp32(E[tok[t]]) and h[t] = bf16(rmsnorm(x[t]) * g): the embedding
// gather fused with the first layer's attention norm.
__global__ __launch_bounds__(256) void embed_rmsnorm_kernel(const int32_t *tok, const uint16_t *E,
                                                            const uint16_t *g, float *x, uint16_t *h, int d,
                                                            float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const uint16_t *src = E + (size_t)tok[t] * d;
  float *xr = x + (size_t)t * d;
  const int nv4 = d / 4;
  float4 v[NORM_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c >= nv4) break;
    const uint2 w = *(const uint2 *)(src + c * 4);
    v[j] = make_float4(lo_bf(w.x), hi_bf(w.x), lo_bf(w.y), hi_bf(w.y));
    *(float4 *)(xr + c * 4) = v[j];
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = block_sum_256(ss, red);
  norm_write_bf16(v, g, h + (size_t)t * d, nv4, 1.f / sqrtf(ss / (float)d + eps));
}

// h[row] = bf16(x[row] / sqrt(mean(x[row]^2) + eps) * g); 256 threads per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, const uint16_t *g, uint16_t *h,
                                                      int d, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float *xr = x + (size_t)t * d;
  const int nv4 = d / 4;
  float4 v[NORM_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c >= nv4) break;
    v[j] = *(const float4 *)(xr + c * 4);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = block_sum_256(ss, red);
  norm_write_bf16(v, g, h + (size_t)t * d, nv4, 1.f / sqrtf(ss / (float)d + eps));
}

// Rotate-half RoPE on q (in place) and k, then append k and v of every row
// at its KV slot.  The row's angles pos * inv_freq[i] are formed in fp64
// once (cos/sin staged in LDS); each thread then rotates 8 consecutive
// pairs with 16-byte loads and stores.
// Cache layout: [page][kv_head][slot_in_page][head_dim].
__global__ __launch_bounds__(256) void rope_kv_kernel(uint16_t *qkv, const int32_t *pos,
                                                      const int32_t *slot, const double *inv_freq,
                                                      uint16_t *kc, uint16_t *vc, int Hq, int Hkv,
                                                      int hd, int ps) {
  __shared__ float cs[64], sn[64];
  const int t = blockIdx.x;
  const int half = hd / 2;
  if ((int)threadIdx.x < half) {
    const double ang = (double)pos[t] * inv_freq[threadIdx.x];
    cs[threadIdx.x] = (float)cos(ang);
    sn[threadIdx.x] = (float)sin(ang);
  }
  __syncthreads();
  const int ld = (Hq + 2 * Hkv) * hd;
  uint16_t *row = qkv + (size_t)t * ld;
  const int s = slot[t];
  const int page = s / ps, off = s % ps;
  const int gph = half / 8;  // groups of 8 pairs per head
  for (int w = threadIdx.x; w < (Hq + Hkv) * gph; w += blockDim.x) {
    const int head = w / gph, i0 = (w % gph) * 8;
    uint16_t *base = row + head * hd;
    const u32x4_t a = *(const u32x4_t *)(base + i0);
    const u32x4_t b = *(const u32x4_t *)(base + half + i0);
    u32x4_t oa, ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + 2 * e;
      const float a0 = lo_bf(a[e]), a1 = hi_bf(a[e]), b0 = lo_bf(b[e]), b1 = hi_bf(b[e]);
      oa[e] = pack_bf2(a0 * cs[i] - b0 * sn[i], a1 * cs[i + 1] - b1 * sn[i + 1]);
      ob[e] = pack_bf2(b0 * cs[i] + a0 * sn[i], b1 * cs[i + 1] + a1 * sn[i + 1]);
    }
    if (head < Hq) {
      *(u32x4_t *)(base + i0) = oa;
      *(u32x4_t *)(base + half + i0) = ob;
    } else {
      uint16_t *dst = kc + (((size_t)page * Hkv + (head - Hq)) * ps + off) * hd;
      *(u32x4_t *)(dst + i0) = oa;
      *(u32x4_t *)(dst + half + i0) = ob;
    }
  }
  const uint16_t *vsrc = row + (Hq + Hkv) * hd;
  for (int w = threadIdx.x; w < Hkv * hd / 8; w += blockDim.x) {
    const int g = (w * 8) / hd, e = (w * 8) % hd;
    *(u32x4_t *)(vc + (((size_t)page * Hkv + g) * ps + off) * hd + e) = *(const u32x4_t *)(vsrc + w * 8);
  }
}

// The step's rotation table for the QKV projection's epilogue: row t holds
// cos(pos[t] * inv_freq[i]) for i < hd/2, then the sines; the angles are
// formed in fp64 as in rope_kv_kernel, so both paths rotate by the same
// fp32 values.  One table serves every layer of the step.
__global__ __launch_bounds__(64) void rope_table_kernel(const int32_t *pos, const double *inv_freq, float *cs,
                                                        int hd) {
  const int t = blockIdx.x, half = hd / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = (double)pos[t] * inv_freq[i];
    cs[(size_t)t * hd + i] = (float)cos(ang);
    cs[(size_t)t * hd + half + i] = (float)sin(ang);
  }
}

// Final RMSNorm for the rows the outputs need: blocks [0, n_embed) take the
// 1/rms of embedding rows (emb_rows[b], or row b when emb_rows is null) into
// rs at their row, which the pooler applies to the residual rows as it
// reads them (no normalised copy of the rows is written); blocks
// [n_embed, n_embed + n_logit) normalise logit_rows[] into hl (bf16,
// LM-head input).
__global__ __launch_bounds__(256) void final_norm_kernel(const float *x, const uint16_t *g,
                                                         const int32_t *logit_rows, const int32_t *emb_rows,
                                                         int n_embed, float *rs, uint16_t *hl, int d, float eps) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const bool emb = b < n_embed;
  const int row = emb ? (emb_rows ? emb_rows[b] : b) : logit_rows[b - n_embed];
  const float *xr = x + (size_t)row * d;
  const int nv4 = d / 4;
  float4 v[NORM_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int c = threadIdx.x + j * 256;
    if (c >= nv4) break;
    v[j] = *(const float4 *)(xr + c * 4);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = block_sum_256(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  if (!emb) {
    norm_write_bf16(v, g, hl + (size_t)(b - n_embed) * d, nv4, inv);
    return;
  }
  if (threadIdx.x == 0) rs[row] = inv;
}

// Segmented pooling.  Segment s = (row0, n, slot, kind, first, last, ctx,
// out).  Grid (segment, block of 256 columns); lane l of each wave owns
// columns 4l .. 4l+3 of the block (16-byte loads, 1 KB per wave per row)
// and wave w sums rows w, w+4, ...; the four waves' sums meet in LDS.  The
// weight total wsum is read here and updated by pool_wsum_kernel
// afterwards so no block reads a value another block has already advanced.
// d is a multiple of 8, so a column group never straddles the row end
// except as a whole.
// The pooled hidden state is the final norm's output (Efficient Iterative
// Retrieval with Heterogeneous Batching, §3.2: the output kernels work on
// the contiguous slice of their item type, with no gather or intermediate
// copy).  SCALED: the pooler reads the item's slice of the residual stream
// and applies the final norm there, (x rs[row]) g[col], the same products
// in the same order as the norm itself; otherwise src rows are already
// normalised (the fp32 path).
template <bool SCALED>
__global__ __launch_bounds__(256) void pool_kernel(const float *src, const float *rs, const uint16_t *g,
                                                   const int32_t *segs, float *sum, const float *wsum, float *kept,
                                                   float *buf, int buf_rows, float *emb, int d) {
  __shared__ float4 part[4][64];
  const int32_t *sg = segs + blockIdx.x * 8;
  const int row0 = sg[0], n = sg[1], slot = sg[2], kind = sg[3] & ~ORTHRUS_POOL_L2;
  const int first = sg[4], last = sg[5], ctx = sg[6], out = sg[7];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.y * 256 + lane * 4;  // first of this lane's 4 columns
  const bool cols = j < d;
  float gc[4] = {1.f, 1.f, 1.f, 1.f};
  if (SCALED && cols) {
    const uint2 gw = *(const uint2 *)(g + j);
    gc[0] = lo_bf(gw.x); gc[1] = hi_bf(gw.x); gc[2] = lo_bf(gw.y); gc[3] = hi_bf(gw.y);
  }
  // the final norm's output at row row0 + r, this lane's 4 columns
  auto rowv = [&](int r) -> float4 {
    const float4 v = *(const float4 *)(src + (size_t)(row0 + r) * d + j);
    if (!SCALED) return v;
    const float inv = rs[row0 + r];
    return make_float4(v.x * inv * gc[0], v.y * inv * gc[1], v.z * inv * gc[2], v.w * inv * gc[3]);
  };
  if (kind == ORTHRUS_POOL_BUFFER) {
    // Keep this chunk's rows at their positions; on the last chunk run the
    // head over all N rows.  Wave w owns the positions p = w (mod 4) and
    // sums them in increasing p, buffered rows (p < ctx) first, then this
    // chunk's rows as it copies them; the waves meet in a fixed order, so
    // the summation order depends on N alone.
    float *bs = buf + (size_t)slot * buf_rows * d + j;
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cols) {
      if (last) {
#pragma unroll 4
        for (int p = wave; p < ctx; p += 4) {
          const float4 v = *(const float4 *)(bs + (size_t)p * d);
          s4.x += v.x;
          s4.y += v.y;
          s4.z += v.z;
          s4.w += v.w;
        }
      }
      const int p0 = ctx + ((wave - ctx) & 3);   // first position >= ctx with p = wave (mod 4)
#pragma unroll 4
      for (int p = p0; p < ctx + n; p += 4) {
        const float4 v = rowv(p - ctx);
        *(float4 *)(bs + (size_t)p * d) = v;
        s4.x += v.x;
        s4.y += v.y;
        s4.z += v.z;
        s4.w += v.w;
      }
    }
    if (!last) return;
    part[wave][lane] = s4;
    __syncthreads();
    if (wave != 0 || !cols) return;
    const int N = ctx + n;
    const float4 a = part[0][lane], b = part[1][lane], c = part[2][lane], e = part[3][lane];
    const float fN = (float)N;
    float *o = emb + (size_t)out * d + j;
    o[0] = (((a.x + b.x) + c.x) + e.x) / fN;
    o[1] = (((a.y + b.y) + c.y) + e.y) / fN;
    o[2] = (((a.z + b.z) + c.z) + e.z) / fN;
    o[3] = (((a.w + b.w) + c.w) + e.w) / fN;
    return;
  }
  if (kind == ORTHRUS_POOL_MEAN || kind == ORTHRUS_POOL_WMEAN) {
    float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cols) {
#pragma unroll 4
      for (int r = wave; r < n; r += 4) {
        const float4 v = rowv(r);
        const float wgt = kind == ORTHRUS_POOL_MEAN ? 1.f : (float)(ctx + r + 1);
        s4.x += wgt * v.x;
        s4.y += wgt * v.y;
        s4.z += wgt * v.z;
        s4.w += wgt * v.w;
      }
    }
    part[wave][lane] = s4;
    __syncthreads();
    if (wave != 0 || !cols) return;
    const float4 a = part[0][lane], b = part[1][lane], c = part[2][lane], e = part[3][lane];
    float tot[4] = {a.x + b.x + c.x + e.x, a.y + b.y + c.y + e.y, a.z + b.z + c.z + e.z, a.w + b.w + c.w + e.w};
    float *sp = sum + (size_t)slot * d + j;
    const long long n64 = n, c64 = ctx;
    const long long add = kind == ORTHRUS_POOL_MEAN ? n64 : n64 * c64 + n64 * (n64 + 1) / 2;
    const float wt = (first ? 0.f : wsum[slot]) + (float)add;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tot[q] += first ? 0.f : sp[q];
      sp[q] = tot[q];
      if (last) emb[(size_t)out * d + j + q] = tot[q] / wt;
    }
  } else {
    if (wave != 0 || !cols) return;
    float *k = kept + (size_t)slot * d + j;
    const bool take = kind != ORTHRUS_POOL_CLS || first;
    if (take) {
      const float4 v = rowv(kind == ORTHRUS_POOL_CLS ? 0 : n - 1);
      k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
    }
    if (last)
#pragma unroll
      for (int q = 0; q < 4; ++q) emb[(size_t)out * d + j + q] = k[q];
  }
}

__global__ void pool_wsum_kernel(const int32_t *segs, int n_segs, float *wsum) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_segs) return;
  const int32_t *sg = segs + s * 8;
  const int n = sg[1], slot = sg[2], kind = sg[3] & ~ORTHRUS_POOL_L2, first = sg[4], ctx = sg[6];
  if (kind != ORTHRUS_POOL_MEAN && kind != ORTHRUS_POOL_WMEAN) {
    if (first) wsum[slot] = 0.f;
    return;
  }
  const long long n64 = n, c64 = ctx;
  const long long add = kind == ORTHRUS_POOL_MEAN ? n64 : n64 * c64 + n64 * (n64 + 1) / 2;
  wsum[slot] = (first ? 0.f : wsum[slot]) + (float)add;
}

// Unit L2 length for the finished embeddings whose pool kind carries the
// L2 flag: one block per segment, e / max(|e|, 1e-12) with the sum of
// squares accumulated in fp32.
__global__ __launch_bounds__(256) void pool_l2_kernel(const int32_t *segs, float *emb, int d) {
  __shared__ float red[4];
  const int32_t *sg = segs + blockIdx.x * 8;
  if (!(sg[3] & ORTHRUS_POOL_L2) || !sg[5]) return;
  float *e = emb + (size_t)sg[7] * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const float4 v = *(const float4 *)(e + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  const float tot = block_sum_256(ss, red);
  const float sc = 1.f / fmaxf(sqrtf(tot), 1e-12f);
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 v = *(const float4 *)(e + c);
    v.x *= sc;
    v.y *= sc;
    v.z *= sc;
    v.w *= sc;
    *(float4 *)(e + c) = v;
  }
}

int launch_embed_rmsnorm(const int32_t *tok, const uint16_t *E, const uint16_t *g, float *x, uint16_t *h, int T,
                         int d, float eps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(embed_rmsnorm_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, tok, E, g, x, h, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_rmsnorm(const float *x, const uint16_t *g, uint16_t *h, int T, int d, float eps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, x, g, h, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_rope_table(const int32_t *pos, const double *inv_freq, float *cs, int T, int hd, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rope_table_kernel, dim3(T), dim3(64), 0, (hipStream_t)stream, pos, inv_freq, cs, hd);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_rope_kv(uint16_t *qkv, const int32_t *pos, const int32_t *slot, const double *inv_freq,
                   uint16_t *kc, uint16_t *vc, int T, int Hq, int Hkv, int hd, int ps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rope_kv_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, qkv, pos, slot,
                     inv_freq, kc, vc, Hq, Hkv, hd, ps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_final_norm(const float *x, const uint16_t *g, const int32_t *logit_rows, const int32_t *emb_rows,
                      int n_embed, int n_logit, float *rs, uint16_t *hl, int d, float eps, void *stream) {
  if (n_embed + n_logit <= 0) return 0;
  hipLaunchKernelGGL(final_norm_kernel, dim3(n_embed + n_logit), dim3(256), 0, (hipStream_t)stream, x,
                     g, logit_rows, emb_rows, n_embed, rs, hl, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_pool(const float *src, const float *rs, const uint16_t *g, const int32_t *segs, int n_segs, float *sum,
                float *wsum, float *kept, float *buf, int buf_rows, float *emb, int d, bool any_l2, void *stream) {
  if (n_segs <= 0) return 0;
  const dim3 grid(n_segs, (d + 255) / 256);
  if (rs)
    hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(256), 0, (hipStream_t)stream, src, rs, g, segs, sum, wsum,
                       kept, buf, buf_rows, emb, d);
  else
    hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(256), 0, (hipStream_t)stream, src, rs, g, segs, sum, wsum,
                       kept, buf, buf_rows, emb, d);
  ORTHRUS_LAUNCH_CHECK();
  hipLaunchKernelGGL(pool_wsum_kernel, dim3((n_segs + 63) / 64), dim3(64), 0, (hipStream_t)stream, segs,
                     n_segs, wsum);
  ORTHRUS_LAUNCH_CHECK();
  if (any_l2) {  // some segment's head carries ORTHRUS_POOL_L2
    hipLaunchKernelGGL(pool_l2_kernel, dim3(n_segs), dim3(256), 0, (hipStream_t)stream, segs, emb, d);
    ORTHRUS_LAUNCH_CHECK();
  }
  return 0;
}

}  // namespace orthrus

namespace orthrus {

// Adapter shrink U = bf16(s * X A^T) for the embedding rows (the LoRA "A"
// projection; Efficient Iterative Retrieval with Heterogeneous Batching,
// §2.2 Parameter sharing): a GEMM with few output columns (3 x rank) and a
// long K.  With one workgroup per 64 x 64 tile, 7168 rows give only 112
// workgroups, each streaming its rows over all of K, which leaves most of
// the chip idle; so K is split over enough workgroups per tile to reach
// one workgroup per slot of the chip, each storing fp32 partial sums, and a second kernel adds the
// splits in order, scales and rounds once.  Without a workspace the scale
// is folded into the GEMM's bf16 epilogue instead.  (A streaming kernel that
// split K over four waves with a deep register ring measured slower on
// MI355X: 37 us against 15 us for 7168 x 48 x 4096.)
static int lora_shrink_splits(int rows, int nr, int K) {
  const int tiles = ((rows + 63) / 64) * ((nr + 63) / 64);
  const int nk = (K + 63) / 64;
  // one round: two 64 x 64 workgroups fit a CU (64 KB of LDS each), and a
  // split count that spills past the slots doubles the launch (7168 rows:
  // 5 splits of 112 tiles ran 22 us, 4 splits fill 448 of 512 slots)
  int s = 2 * gemm_cu_count() / tiles;
  s = std::min(s, std::min(8, nk / 4));
  return std::max(s, 1);
}

size_t lora_shrink_ws_bytes(int rows, int nr, int K) {
  const int s = lora_shrink_splits(rows, nr, K);
  return s > 1 ? (size_t)s * rows * nr * 4 : 0;
}

// U[e] = bf16(scale * (P[0][e] + P[1][e] + ...)), e over rows * nr elements
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(const float *P, int splits, size_t n, float scale,
                                                            uint16_t *U) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    float acc = P[e];
    for (int y = 1; y < splits; ++y) acc += P[(size_t)y * n + e];
    U[e] = (uint16_t)f2bf(scale * acc);
  }
}

int launch_lora_shrink(const uint16_t *X, int ldx, const uint16_t *A, int rows, int nr, int K, float scale,
                       uint16_t *U, float *ws, size_t ws_bytes, void *stream) {
  if (rows <= 0 || nr <= 0) return 0;
  const int splits = lora_shrink_splits(rows, nr, K);
  if (splits < 2 || !ws || ws_bytes < lora_shrink_ws_bytes(rows, nr, K))
    return launch_gemm(X, ldx, A, K, U, nr, rows, nr, K, EPI_BF16, 0, scale, nullptr, stream);
  if (int r = launch_gemm_f32_ksplit(X, ldx, A, K, ws, rows, nr, K, splits, stream)) return r;
  const size_t n = (size_t)rows * nr;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(ksplit_reduce_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, ws, splits, n, scale, U);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus

namespace orthrus {

// Seeded synthetic bf16 values from the SplitMix64 counter hash (Steele,
// Lea and Flood 2014): value i of (seed, tensor_id) is
//   z = ((seed << 32) ^ tensor_id) + (i + 1) * 0x9E3779B97F4A7C15
//   z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB
//   h = z ^ (z >> 31); u = (h >> 40) * 2^-24; v = bf16_rne((2u - 1) * 1.7320508f)
// Every step is exact integer arithmetic or one correctly rounded fp32
// operation, so any implementation of the definition gives the same bits.
__global__ void hash_fill_kernel(uint16_t *dst, uint64_t n, uint64_t key, uint64_t start) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    uint64_t z = key + (start + i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z = z ^ (z >> 31);
    const float u = (float)(uint32_t)(z >> 40) * (1.0f / 16777216.0f);
    const float t = 2.0f * u - 1.0f;   // exact
    dst[i] = (uint16_t)f2bf(__fmul_rn(t, 1.7320508f));
  }
}

int launch_hash_fill(uint16_t *dst, uint64_t n, uint32_t seed, uint32_t tensor_id, uint64_t start, void *stream) {
  if (n == 0) return 0;
  const uint64_t key = ((uint64_t)seed << 32) ^ (uint64_t)tensor_id;
  hipLaunchKernelGGL(hash_fill_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, dst, n, key, start);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus
