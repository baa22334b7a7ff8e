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

namespace orthrus {

// x[t, :] = fp32(E[tok[t], :]); one workgroup per row, 8 values per chunk.
__global__ void embed_gather_kernel(const int32_t *tok, const uint16_t *E, float *x, int d) {
  const int t = blockIdx.x;
  const uint16_t *src = E + (size_t)tok[t] * d;
  float *dst = x + (size_t)t * d;
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const u32x4_t w = *(const u32x4_t *)(src + c * 8);
    float4 a = make_float4(lo_bf(w[0]), hi_bf(w[0]), lo_bf(w[1]), hi_bf(w[1]));
    float4 b = make_float4(lo_bf(w[2]), hi_bf(w[2]), lo_bf(w[3]), hi_bf(w[3]));
    *(float4 *)(dst + c * 8) = a;
    *(float4 *)(dst + c * 8 + 4) = b;
  }
}

__device__ __forceinline__ float block_sum_256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
  __syncthreads();
  return s;
}

// h[row] = bf16(x[row] / sqrt(mean(x[row]^2) + eps) * g); 256 threads per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *x, const uint16_t *g, uint16_t *h,
                                                      int d, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const float *xr = x + (size_t)t * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    const float4 v = *(const float4 *)(xr + c * 4);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum_256(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  uint16_t *hr = h + (size_t)t * d;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    const float4 v = *(const float4 *)(xr + c * 4);
    const uint2 gw = *(const uint2 *)(g + c * 4);
    uint2 o;
    o.x = pack_bf2(v.x * inv * lo_bf(gw.x), v.y * inv * hi_bf(gw.x));
    o.y = pack_bf2(v.z * inv * lo_bf(gw.y), v.w * inv * hi_bf(gw.y));
    *(uint2 *)(hr + c * 4) = o;
  }
}

// Rotate-half RoPE on q (in place) and k, then append k and v of every row
// at its KV slot.  Angles pos * inv_freq[i] are formed in fp64.
// Cache layout: [page][kv_head][slot_in_page][head_dim].
__global__ __launch_bounds__(256) void rope_kv_kernel(uint16_t *qkv, const int32_t *pos,
                                                      const int32_t *slot, const double *inv_freq,
                                                      uint16_t *kc, uint16_t *vc, int Hq, int Hkv,
                                                      int hd, int ps) {
  const int t = blockIdx.x;
  const int half = hd / 2;
  const int ld = (Hq + 2 * Hkv) * hd;
  uint16_t *row = qkv + (size_t)t * ld;
  const double p = (double)pos[t];
  const int s = slot[t];
  const int page = s / ps, off = s % ps;
  // q and k heads: one (head, pair) per thread iteration
  const int n_rot = (Hq + Hkv) * half;
  for (int w = threadIdx.x; w < n_rot; w += blockDim.x) {
    const int head = w / half, i = w % half;
    const double ang = p * inv_freq[i];
    const float c = (float)cos(ang), sn = (float)sin(ang);
    uint16_t *base = row + head * hd;
    const float x1 = bf2f(base[i]), x2 = bf2f(base[i + half]);
    const uint16_t o1 = (uint16_t)f2bf(x1 * c - x2 * sn);
    const uint16_t o2 = (uint16_t)f2bf(x2 * c + x1 * sn);
    if (head < Hq) {
      base[i] = o1;
      base[i + half] = o2;
    } else {
      const int g = head - Hq;
      uint16_t *dst = kc + (((size_t)page * Hkv + g) * ps + off) * hd;
      dst[i] = o1;
      dst[i + half] = o2;
    }
  }
  const uint16_t *vsrc = row + (Hq + Hkv) * hd;
  for (int w = threadIdx.x; w < Hkv * hd; w += blockDim.x) {
    const int g = w / hd, e = w % hd;
    vc[(((size_t)page * Hkv + g) * ps + off) * hd + e] = vsrc[w];
  }
}

// Final RMSNorm for the rows the outputs need: blocks [0, n_embed) normalise
// embedding rows into hf (fp32, pooler input); blocks [n_embed, n_embed +
// n_logit) normalise logit_rows[] into hl (bf16, LM-head input).
__global__ __launch_bounds__(256) void final_norm_kernel(const float *x, const uint16_t *g,
                                                         const int32_t *logit_rows, int n_embed,
                                                         float *hf, uint16_t *hl, int d, float eps) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const bool emb = b < n_embed;
  const int row = emb ? b : logit_rows[b - n_embed];
  const float *xr = x + (size_t)row * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    const float4 v = *(const float4 *)(xr + c * 4);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum_256(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    const float4 v = *(const float4 *)(xr + c * 4);
    const uint2 gw = *(const uint2 *)(g + c * 4);
    const float4 o = make_float4(v.x * inv * lo_bf(gw.x), v.y * inv * hi_bf(gw.x),
                                 v.z * inv * lo_bf(gw.y), v.w * inv * hi_bf(gw.y));
    if (emb) {
      *(float4 *)(hf + (size_t)b * d + c * 4) = o;
    } else {
      uint2 w;
      w.x = pack_bf2(o.x, o.y);
      w.y = pack_bf2(o.z, o.w);
      *(uint2 *)(hl + (size_t)(b - n_embed) * d + c * 4) = w;
    }
  }
}

// Segmented pooling.  Segment s = (row0, n, slot, kind, first, last, ctx,
// out).  Grid (segment, column block); each thread owns one column and walks
// the segment's rows in order.  The weight total wsum is read here and
// updated by pool_wsum_kernel afterwards so no block reads a value another
// block has already advanced.
__global__ __launch_bounds__(256) void pool_kernel(const float *hf, const int32_t *segs, float *sum,
                                                   const float *wsum, float *kept, float *emb,
                                                   int d) {
  const int32_t *sg = segs + blockIdx.x * 8;
  const int row0 = sg[0], n = sg[1], slot = sg[2], kind = sg[3];
  const int first = sg[4], last = sg[5], ctx = sg[6], out = sg[7];
  const int j = blockIdx.y * blockDim.x + threadIdx.x;
  if (j >= d) return;
  const float *col = hf + (size_t)row0 * d + j;
  if (kind == ORTHRUS_POOL_MEAN || kind == ORTHRUS_POOL_WMEAN) {
    float s = 0.f;
    if (kind == ORTHRUS_POOL_MEAN) {
      for (int r = 0; r < n; ++r) s += col[(size_t)r * d];
    } else {
      for (int r = 0; r < n; ++r) s += (float)(ctx + r + 1) * col[(size_t)r * d];
    }
    const float prev = first ? 0.f : sum[(size_t)slot * d + j];
    const float tot = prev + s;
    sum[(size_t)slot * d + j] = tot;
    if (last) {
      const long long n64 = n, c64 = ctx;
      const long long add = kind == ORTHRUS_POOL_MEAN ? n64 : n64 * c64 + n64 * (n64 + 1) / 2;
      const float wt = (first ? 0.f : wsum[slot]) + (float)add;
      emb[(size_t)out * d + j] = tot / wt;
    }
  } else {
    float *k = kept + (size_t)slot * d + j;
    if (kind == ORTHRUS_POOL_CLS) {
      if (first) *k = col[0];
    } else {
      *k = col[(size_t)(n - 1) * d];
    }
    if (last) emb[(size_t)out * d + j] = *k;
  }
}

__global__ void pool_wsum_kernel(const int32_t *segs, int n_segs, float *wsum) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_segs) return;
  const int32_t *sg = segs + s * 8;
  const int n = sg[1], slot = sg[2], kind = sg[3], first = sg[4], ctx = sg[6];
  if (kind != ORTHRUS_POOL_MEAN && kind != ORTHRUS_POOL_WMEAN) {
    if (first) wsum[slot] = 0.f;
    return;
  }
  const long long n64 = n, c64 = ctx;
  const long long add = kind == ORTHRUS_POOL_MEAN ? n64 : n64 * c64 + n64 * (n64 + 1) / 2;
  wsum[slot] = (first ? 0.f : wsum[slot]) + (float)add;
}

int launch_embed_gather(const int32_t *tok, const uint16_t *E, float *x, int T, int d, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(embed_gather_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, tok, E, x, d);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_rmsnorm(const float *x, const uint16_t *g, uint16_t *h, int T, int d, float eps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, x, g, h, d, eps);
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

int launch_final_norm(const float *x, const uint16_t *g, const int32_t *logit_rows, int n_embed,
                      int n_logit, float *hf, uint16_t *hl, int d, float eps, void *stream) {
  if (n_embed + n_logit <= 0) return 0;
  hipLaunchKernelGGL(final_norm_kernel, dim3(n_embed + n_logit), dim3(256), 0, (hipStream_t)stream, x,
                     g, logit_rows, n_embed, hf, hl, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_pool(const float *hf, const int32_t *segs, int n_segs, float *sum, float *wsum, float *kept,
                float *emb, int d, void *stream) {
  if (n_segs <= 0) return 0;
  hipLaunchKernelGGL(pool_kernel, dim3(n_segs, (d + 255) / 256), dim3(256), 0, (hipStream_t)stream, hf,
                     segs, sum, wsum, kept, emb, d);
  ORTHRUS_LAUNCH_CHECK();
  hipLaunchKernelGGL(pool_wsum_kernel, dim3((n_segs + 63) / 64), dim3(64), 0, (hipStream_t)stream, segs,
                     n_segs, wsum);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus
