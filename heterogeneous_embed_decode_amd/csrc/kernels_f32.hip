// fp32 path of the step (orthrus_model_cfg.dtype == ORTHRUS_F32): weights,
// KV pages, activations and accumulations all in fp32, for models whose
// reference numerics are fp32 (the tiny decoder).  The same forward as the
// bf16 path (Efficient Iterative Retrieval with Heterogeneous Batching,
// §3.1: one shared forward over every row; §3.2: embedding chunks, prefill
// chunks and decode rows in one batch; §2.2 Parameter sharing: the adapter
// on embedding rows only), written for correctness at small sizes rather
// than speed: a tiled FMA GEMM with the step's epilogues and the adapter's
// expand, row-parallel norms, RoPE with fp64 angles, and one workgroup per
// (row, query head) for attention over the paged cache with an fp32 online
// softmax.
#include "device_common.h"
#include "orthrus_internal.h"

namespace orthrus {

// ---- GEMM: C = alpha * A B^T (+ adapter), fp32 --------------------------
// 64 x 64 output tile, 256 threads as 16 x 16, each thread 4 x 4 outputs;
// K in steps of 16 staged transposed in LDS.  SwiGLU: B holds gate rows
// 0..N-1 and up rows b_up_row..; the thread keeps both accumulators.
// Adapter (rows < lrows): acc += sum_k U[m][sec(n) * r + k] * Bx[n][k], where
// column n is in section 0 below sec1, 1 below sec2, else 2.
struct GemmF32Args {
  const float *A, *B;
  float *C;
  int lda, ldb, ldc, M, N, K, b_up_row, epi;
  float alpha;
  const float *U, *Bx;
  int ldu, r, lrows, sec1, sec2;
};

constexpr int F32_TILE = 64, F32_BK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
  __shared__ float As[F32_BK][F32_TILE + 4];
  __shared__ float Bs[2][F32_BK][F32_TILE + 4];
  const bool dual = g.epi == EPI_SWIGLU;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.y * F32_TILE, n0 = blockIdx.x * F32_TILE;
  float acc[2][4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += F32_BK) {
    // 64 rows x 16 k per operand: each thread loads 4 values
    for (int e = threadIdx.x; e < F32_TILE * F32_BK; e += 256) {
      const int rr = e / F32_BK, kk = e % F32_BK;
      const int m = m0 + rr, n = n0 + rr, k = k0 + kk;
      As[kk][rr] = (m < g.M && k < g.K) ? g.A[(size_t)m * g.lda + k] : 0.f;
      Bs[0][kk][rr] = (n < g.N && k < g.K) ? g.B[(size_t)n * g.ldb + k] : 0.f;
      if (dual) Bs[1][kk][rr] = (n < g.N && k < g.K) ? g.B[(size_t)(g.b_up_row + n) * g.ldb + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F32_BK; ++kk) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[0][kk][tx * 4 + i];
        u[i] = dual ? Bs[1][kk][tx * 4 + i] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][i][j] = fmaf(a[i], b[j], acc[0][i][j]);
          if (dual) acc[1][i][j] = fmaf(a[i], u[j], acc[1][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float v = acc[0][i][j];
      if (g.U && m < g.lrows) {
        const int sec = n < g.sec1 ? 0 : (n < g.sec2 ? 1 : 2);
        const float *ur = g.U + (size_t)m * g.ldu + sec * g.r;
        const float *br = g.Bx + (size_t)n * g.r;
        float d = 0.f;
        for (int k = 0; k < g.r; ++k) d = fmaf(ur[k], br[k], d);
        v += d;
      }
      float *c = g.C + (size_t)m * g.ldc + n;
      if (g.epi == EPI_RESID) {
        *c += v;
      } else if (dual) {
        const float up = acc[1][i][j];
        *c = v / (1.f + expf(-v)) * up;
      } else {
        *c = g.alpha * v;
      }
    }
  }
}

int launch_gemm_f32(const float *A, int lda, const float *B, int ldb, float *C, int ldc, int M, int N, int K,
                    int epi, int b_up_row, float alpha, const float *U, int ldu, const float *Bx, int r, int lrows,
                    int sec1, int sec2, void *stream) {
  if (M <= 0 || N <= 0) return 0;
  GemmF32Args g{A, B, C, lda, ldb, ldc, M, N, K, b_up_row, epi, alpha, U, Bx, ldu, r, lrows, sec1, sec2};
  dim3 grid((N + F32_TILE - 1) / F32_TILE, (M + F32_TILE - 1) / F32_TILE);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, (hipStream_t)stream, g);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

// ---- norms ---------------------------------------------------------------
__device__ __forceinline__ float block_sum_f32(float v, float *red) {
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

// h[t] = x[t] / sqrt(mean(x[t]^2) + eps) * g; with tok, x[t] = E[tok[t]]
// first (the embedding gather).  One workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_f32_kernel(const int32_t *tok, const float *E, float *x,
                                                          const float *g, float *h, int d, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float *xr = x + (size_t)t * d;
  if (tok) {
    const float *er = E + (size_t)tok[t] * d;
    for (int c = threadIdx.x; c < d; c += 256) xr[c] = er[c];
    __syncthreads();
  }
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) ss = fmaf(xr[c], xr[c], ss);
  ss = block_sum_f32(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += 256) h[(size_t)t * d + c] = xr[c] * inv * g[c];
}

int launch_rmsnorm_f32(const int32_t *tok, const float *E, float *x, const float *g, float *h, int T, int d,
                       float eps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rmsnorm_f32_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, tok, E, x, g, h, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

// Final norm: blocks [0, n_embed) write hf at rows 0..n_embed-1 (the
// embedding slice, pooler input); blocks [n_embed, n_embed + n_logit) write
// hl[k] for logit_rows[k] (LM-head input).
__global__ __launch_bounds__(256) void final_norm_f32_kernel(const float *x, const float *g,
                                                             const int32_t *logit_rows, int n_embed, float *hf,
                                                             float *hl, int d, float eps) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const bool emb = b < n_embed;
  const int row = emb ? b : logit_rows[b - n_embed];
  const float *xr = x + (size_t)row * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) ss = fmaf(xr[c], xr[c], ss);
  ss = block_sum_f32(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  float *dst = emb ? hf + (size_t)row * d : hl + (size_t)(b - n_embed) * d;
  for (int c = threadIdx.x; c < d; c += 256) dst[c] = xr[c] * inv * g[c];
}

int launch_final_norm_f32(const float *x, const float *g, const int32_t *logit_rows, int n_embed, int n_logit,
                          float *hf, float *hl, int d, float eps, void *stream) {
  if (n_embed + n_logit <= 0) return 0;
  hipLaunchKernelGGL(final_norm_f32_kernel, dim3(n_embed + n_logit), dim3(256), 0, (hipStream_t)stream, x, g,
                     logit_rows, n_embed, hf, hl, d, eps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

// ---- RoPE + KV append ----------------------------------------------------
// Rotate-half RoPE on every q and k head of row t at position pos[t] (pair i
// = (i, i + hd/2) turned by pos * inv_freq[i], angles in fp64); q in place,
// k and v to the row's cache slot ([page][kv_head][slot][head_dim]).
__global__ __launch_bounds__(256) void rope_kv_f32_kernel(float *qkv, const int32_t *pos, const int32_t *slot,
                                                          const double *inv_freq, float *kc, float *vc, int Hq,
                                                          int Hkv, int hd, int ps) {
  __shared__ float cs[64], sn[64];
  const int t = blockIdx.x, half = hd / 2;
  if ((int)threadIdx.x < half) {
    const double ang = (double)pos[t] * inv_freq[threadIdx.x];
    cs[threadIdx.x] = (float)cos(ang);
    sn[threadIdx.x] = (float)sin(ang);
  }
  __syncthreads();
  float *row = qkv + (size_t)t * (Hq + 2 * Hkv) * hd;
  const int s = slot[t], page = s / ps, off = s % ps;
  for (int w = threadIdx.x; w < (Hq + Hkv) * half; w += blockDim.x) {
    const int head = w / half, i = w % half;
    float *base = row + head * hd;
    const float a = base[i], b = base[i + half];
    const float oa = a * cs[i] - b * sn[i], ob = b * cs[i] + a * sn[i];
    if (head < Hq) {
      base[i] = oa;
      base[i + half] = ob;
    } else {
      float *dst = kc + (((size_t)page * Hkv + (head - Hq)) * ps + off) * hd;
      dst[i] = oa;
      dst[i + half] = ob;
    }
  }
  const float *vsrc = row + (Hq + Hkv) * hd;
  for (int w = threadIdx.x; w < Hkv * hd; w += blockDim.x) {
    const int g = w / hd, e = w % hd;
    vc[(((size_t)page * Hkv + g) * ps + off) * hd + e] = vsrc[w];
  }
}

int launch_rope_kv_f32(float *qkv, const int32_t *pos, const int32_t *slot, const double *inv_freq, float *kc,
                       float *vc, int T, int Hq, int Hkv, int hd, int ps, void *stream) {
  if (T <= 0) return 0;
  hipLaunchKernelGGL(rope_kv_f32_kernel, dim3(T), dim3(256), 0, (hipStream_t)stream, qkv, pos, slot, inv_freq, kc,
                     vc, Hq, Hkv, hd, ps);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

// ---- attention ------------------------------------------------------------
// One 64-lane workgroup per (row t, query head h): keys 0..pos[t] of the
// row's request, read through its page list from KV head h / (Hq/Hkv).
// Blocks of 64 keys: lane j scores key k0 + j, the block maximum and sum
// update the running (m, l), the block's weights go through LDS, and each
// lane accumulates the output dims d = lane, lane + 64.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float *qkv, const float *kc, const float *vc,
                                                      const int32_t *page_ids, const DevItem *items,
                                                      const int32_t *row_item, const int32_t *pos, float *o, int Hq,
                                                      int Hkv, int hd, int ps, float scale) {
  __shared__ float q[128], p[64];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int kvh = h / (Hq / Hkv);
  const DevItem it = items[row_item[t]];
  const int nk = pos[t] + 1;
  const float *qr = qkv + (size_t)t * (Hq + 2 * Hkv) * hd + h * hd;
  for (int d = lane; d < hd; d += 64) q[d] = qr[d];
  __syncthreads();
  auto key_base = [&](const float *cache, int k) {
    const int page = page_ids[it.page_off + k / ps];
    return cache + (((size_t)page * Hkv + kvh) * ps + k % ps) * hd;
  };
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int k = k0 + lane;
    float s = -INFINITY;
    if (k < nk) {
      const float *kr = key_base(kc, k);
      float dot = 0.f;
      for (int d = 0; d < hd; ++d) dot = fmaf(q[d], kr[d], dot);
      s = dot * scale;
    }
    float bm = s;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off, 64));
    const float mn = fmaxf(m, bm);
    const float alpha = expf(m - mn);  // 0 on the first block (m = -inf)
    const float pk = k < nk ? expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(pk);
    p[lane] = pk;
    __syncthreads();
    acc0 *= alpha;
    acc1 *= alpha;
    const int nb = min(64, nk - k0);
    for (int j = 0; j < nb; ++j) {
      const float *vr = key_base(vc, k0 + j);
      if (lane < hd) acc0 = fmaf(p[j], vr[lane], acc0);
      if (lane + 64 < hd) acc1 = fmaf(p[j], vr[lane + 64], acc1);
    }
    __syncthreads();
    m = mn;
  }
  float *orow = o + (size_t)t * Hq * hd + h * hd;
  if (lane < hd) orow[lane] = acc0 / l;
  if (lane + 64 < hd) orow[lane + 64] = acc1 / l;
}

int launch_attn_f32(const float *qkv, const float *kc, const float *vc, const int32_t *page_ids,
                    const DevItem *items, const int32_t *row_item, const int32_t *pos, float *o, int T, int Hq,
                    int Hkv, int hd, int ps, void *stream) {
  if (T <= 0) return 0;
  const float scale = (float)(1.0 / sqrt((double)hd));
  hipLaunchKernelGGL(attn_f32_kernel, dim3(T, Hq), dim3(64), 0, (hipStream_t)stream, qkv, kc, vc, page_ids, items,
                     row_item, pos, o, Hq, Hkv, hd, ps, scale);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus
