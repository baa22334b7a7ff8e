// Next-token choice on the logit rows of a step: greedy, or temperature
// sampling within a nucleus (top-p); one workgroup per row.
//
// Efficient Iterative Retrieval with Heterogeneous Batching: §3.1 (the emit
// stage hands each generation request's last-row logits to the sampler) and
// §2.2 Generation (one new token per decoding step).  The page fixes no
// sampling rule.  The one computed here turns the logits into integer
// weights, so that the token is a pure function of the logits, the row's
// temperature T and top-p and a caller-supplied 32-bit uniform U:
//   s = fp32(log2 e / T); t_i = (l_i - max) * s in fp32 (0 at the maximum);
//   q_i = floor(2^(30 + t_i)) and 0 below t = -30, where 2^t is
//     2^floor(t) * P(t - floor(t)), P the degree-7 Taylor polynomial of 2^f
//     evaluated by fp32 Horner steps without fused multiply-adds;
//   Z = sum q, P16 = rint(top_p * 2^16) in [1, 2^16], target = ceil(Z P16 / 2^16);
//   tau = the largest weight whose upper set {q >= tau} weighs >= target; the
//     nucleus is every q > tau plus the first ceil((target - mass(q > tau)) / tau)
//     tokens of weight tau in index order;
//   x = floor(mass * U / 2^32); the token is the first, in index order, at
//     which the running nucleus weight exceeds x.
// tau comes from a most-significant-digit-first radix select whose bins
// hold weight sums (digits of 8, 8, 8 and 7 bits from bit 30 down).  The
// first radix pass forms the weights from the logits; when the row's
// weights fit in LDS (vocabularies up to 38400 tokens: 150 KB) they are kept
// there and the later radix passes and the draw read them back, otherwise
// every pass recomputes them from the logits (the later reads from L2).
// Either way the kernel needs no memory beyond its inputs and outputs.
#include "device_common.h"
#include "orthrus_internal.h"

namespace orthrus {
namespace {

// fp32((ln 2)^j / j!), formed in fp64 by repeated multiplication
constexpr float taylor_coef(int j) {
  double c = 1.0;
  for (int i = 1; i <= j; ++i) c = c * 0.69314718055994530942 / i;
  return (float)c;
}
constexpr float TC0 = taylor_coef(0), TC1 = taylor_coef(1), TC2 = taylor_coef(2), TC3 = taylor_coef(3),
                TC4 = taylor_coef(4), TC5 = taylor_coef(5), TC6 = taylor_coef(6), TC7 = taylor_coef(7);

__device__ __forceinline__ uint32_t weight_of(float l, float mx, float s) {
#pragma clang fp contract(off)
  const float d = l - mx;
  const float t = d == 0.f ? 0.f : d * s;
  if (!(t >= -30.f)) return 0u;
  const float k = floorf(t);
  const float f = t - k;
  float p = TC7;
  p = p * f; p = p + TC6;
  p = p * f; p = p + TC5;
  p = p * f; p = p + TC4;
  p = p * f; p = p + TC3;
  p = p * f; p = p + TC2;
  p = p * f; p = p + TC1;
  p = p * f; p = p + TC0;
  return (uint32_t)ldexpf(p, 30 + (int)k);    // exact scaling; p in [1, 2)
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor((unsigned long long)v, o, 64);
  return v;
}

// One DPP step: v from the lane CTRL names (0 where that lane is outside the
// row or the row is not in ROWS).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Inclusive scan across the 64 lanes: row_shr 1, 2, 4, 8 within rows of 16,
// then row_bcast 15 (rows 1, 3) and row_bcast 31 (rows 2, 3).
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  v += dpp_u64<0x111, 0xf>(v);
  v += dpp_u64<0x112, 0xf>(v);
  v += dpp_u64<0x114, 0xf>(v);
  v += dpp_u64<0x118, 0xf>(v);
  v += dpp_u64<0x142, 0xa>(v);
  v += dpp_u64<0x143, 0xc>(v);
  return v;
}

__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Integer target of the nucleus: ceil(Z * P16 / 2^16) without overflow.
__device__ __forceinline__ uint64_t nucleus_target(uint64_t Z, uint64_t P16) {
  return (Z >> 16) * P16 + (((Z & 0xffffull) * P16 + 0xffffull) >> 16);
}

// floor(mass * U / 2^32) without a 128-bit product.
__device__ __forceinline__ uint64_t draw_point(uint64_t mass, uint64_t U) {
  return (mass >> 32) * U + (((mass & 0xffffffffull) * U) >> 32);
}

// One workgroup of SMP_T threads per row.  The max and radix passes read the
// row as groups of 4 consecutive logits, group g = it * SMP_T + tid, with
// SMP_U groups per thread in flight; the draw splits the row into one
// contiguous segment per wave.
constexpr int SMP_T = 1024;
constexpr int SMP_W = SMP_T / 64;
constexpr int SMP_U = 4;
constexpr int SMP_CACHE_GROUPS = 9600;  // groups of 4 weights kept in LDS (150 KB)

__device__ __forceinline__ float4 load4(const float *L, int g, int V, int vec_ok) {
  const int i = 4 * g;
  if (vec_ok && i + 4 <= V) return *(const float4 *)(L + i);
  float4 r;
  r.x = i < V ? L[i] : 0.f;
  r.y = i + 1 < V ? L[i + 1] : 0.f;
  r.z = i + 2 < V ? L[i + 2] : 0.f;
  r.w = i + 3 < V ? L[i + 3] : 0.f;
  return r;
}

// cached: the launch gave 16 n_grp bytes of dynamic LDS for the weights
__global__ __launch_bounds__(SMP_T) void sample_kernel(const float *__restrict__ logits, int64_t ld, int V,
                                                       int vec_ok, const float *__restrict__ temp,
                                                       const float *__restrict__ top_p,
                                                       const uint32_t *__restrict__ uni,
                                                       int32_t *__restrict__ out, int cached) {
  extern __shared__ uint4 qcache[];  // weights of group g (tokens 4g .. 4g+3), zero past V
  __shared__ unsigned long long hist[2][256];
  __shared__ unsigned long long seg_a[SMP_W];
  __shared__ uint32_t seg_c[SMP_W];
  __shared__ float red_m[SMP_W];
  __shared__ int red_i[SMP_W];
  __shared__ unsigned long long s_above, s_target;
  __shared__ uint32_t s_digit;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float *L = logits + (size_t)row * ld;
  const int n_grp = (V + 3) >> 2;
  // the row's parameters, read before the max pass so their latency hides behind it
  const float T = temp ? temp[row] : 0.f;
  const float pf = top_p ? top_p[row] : 1.f;
  const uint64_t U = temp ? uni[row] : 0;

  // Maximum and its first index.  A thread's groups come in increasing
  // index order, so a strict comparison keeps the first.
  float mx = 0.f;
  int ix = -1;
#pragma unroll 1
  for (int g0 = tid; g0 < n_grp; g0 += SMP_U * SMP_T) {
    float4 v[SMP_U];
#pragma unroll
    for (int u = 0; u < SMP_U; ++u) v[u] = load4(L, g0 + u * SMP_T, V, vec_ok);
#pragma unroll
    for (int u = 0; u < SMP_U; ++u) {
      const int i = 4 * (g0 + u * SMP_T);
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (i + c < V && (ix < 0 || e[c] > mx)) { mx = e[c]; ix = i + c; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(ix, o, 64);
    if (oi >= 0 && (ix < 0 || om > mx || (om == mx && oi < ix))) { mx = om; ix = oi; }
  }
  if (lane == 0) { red_m[w] = mx; red_i[w] = ix; }
  if (tid < 256) hist[0][tid] = 0;
  __syncthreads();
  mx = red_m[0];
  ix = red_i[0];
#pragma unroll 1
  for (int j = 1; j < SMP_W; ++j) {
    const float om = red_m[j];
    const int oi = red_i[j];
    if (oi >= 0 && (om > mx || (om == mx && oi < ix))) { mx = om; ix = oi; }
  }
  if (!(T > 0.f)) {                       // greedy (uniform over the workgroup)
    if (tid == 0) out[row] = ix;
    return;
  }
  const float s = (float)(1.4426950408889634 / (double)T);
  const uint64_t P16 = (uint64_t)fminf(fmaxf(rintf(pf * 65536.f), 1.f), 65536.f);

  // Radix select of tau.  `above` is the weight of the tokens whose weight
  // exceeds every remaining candidate; `pref` holds tau's digits so far.
  // Level lev builds its histogram in hist[lev & 1]; wave 0 picks the digit
  // and clears the other buffer for the next level.
  uint64_t above = 0, target = 0;
  uint32_t pref = 0;
#pragma unroll 1
  for (int lev = 0; lev < 4; ++lev) {
    const int hs = lev == 0 ? 31 : 31 - 8 * lev;   // tokens in play: q >> hs == pref
    const int sh = lev == 3 ? 0 : 23 - 8 * lev;     // this digit: bits sh .. hs-1
    const uint32_t mask = (1u << (hs - sh)) - 1u;
    unsigned long long *H = hist[lev & 1];
    uint64_t h0 = 0;                                // digit 0 is summed in registers
#pragma unroll 1
    for (int g0 = tid; g0 < n_grp; g0 += SMP_U * SMP_T) {
      uint32_t qq[SMP_U][4];
      if (cached && lev > 0) {
#pragma unroll
        for (int u = 0; u < SMP_U; ++u) {
          const int gi = g0 + u * SMP_T;
          const uint4 w4 = gi < n_grp ? qcache[gi] : make_uint4(0u, 0u, 0u, 0u);
          qq[u][0] = w4.x; qq[u][1] = w4.y; qq[u][2] = w4.z; qq[u][3] = w4.w;
        }
      } else {
        float4 v[SMP_U];
#pragma unroll
        for (int u = 0; u < SMP_U; ++u) v[u] = load4(L, g0 + u * SMP_T, V, vec_ok);
#pragma unroll
        for (int u = 0; u < SMP_U; ++u) {
          const int i = 4 * (g0 + u * SMP_T);
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) qq[u][c] = i + c < V ? weight_of(e[c], mx, s) : 0u;
          if (cached && g0 + u * SMP_T < n_grp)
            qcache[g0 + u * SMP_T] = make_uint4(qq[u][0], qq[u][1], qq[u][2], qq[u][3]);
        }
      }
#pragma unroll
      for (int u = 0; u < SMP_U; ++u) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t q = qq[u][c];
          const uint32_t dg = (q >> sh) & mask;
          if ((q >> hs) == pref) {
            if (dg == 0) h0 += q;
            else atomicAdd(&H[dg], (unsigned long long)q);
          }
        }
      }
    }
    h0 = wave_sum_u64(h0);
    if (lane == 0 && h0) atomicAdd(&H[0], (unsigned long long)h0);
    __syncthreads();
    if (w == 0) {
      // lane l holds digits 255-4l .. 252-4l, so lane order is descending digit order
      uint64_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = H[255 - 4 * lane - k];
      const uint64_t ls = h[0] + h[1] + h[2] + h[3];
      const uint64_t incl = wave_scan_u64(ls);
      const uint64_t tgt = lev == 0 ? nucleus_target(lane63_u64(incl), P16) : target;
      uint64_t run = above + (incl - ls);           // weight of the in-play digits above h[0]
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (run < tgt && run + h[k] >= tgt) {       // exactly one digit of the wave
          s_digit = 255u - (uint32_t)(4 * lane + k);
          s_above = run;
        }
        run += h[k];
      }
      if (lev == 0 && lane == 0) s_target = tgt;
#pragma unroll
      for (int k = 0; k < 4; ++k) hist[(lev + 1) & 1][4 * lane + k] = 0;
    }
    __syncthreads();
    above = s_above;
    if (lev == 0) target = s_target;
    pref = (pref << (hs - sh)) | s_digit;
  }
  const uint64_t tau = pref;
  const uint64_t n_tie = (target - above + tau - 1) / tau;
  const uint64_t x = draw_point(above + n_tie * tau, U);

  // Draw.  The running nucleus weight at token i is A(i) + tau * min(C(i), n_tie)
  // with A the weight of the tokens above tau and C the number of tokens at
  // tau up to i; the token is the number of tokens whose running weight is
  // <= x.  Wave w owns the contiguous chunks [w * cpw, (w + 1) * cpw) of 256
  // tokens (lane l: tokens 4l .. 4l+3 of a chunk).  Each wave sums its
  // segment; the one wave whose segment crosses x then walks its chunks.
  const int n_chunk = (V + 255) >> 8;
  const int cpw = (n_chunk + SMP_W - 1) / SMP_W;
  const int cb = w * cpw, ce = min(n_chunk, cb + cpw);
  uint64_t sa = 0;
  uint32_t sc = 0;
  // the weights of group g (tokens 4g .. 4g+3; zero past V or for a chunk
  // past the wave's segment)
  auto group_q = [&](int gi, bool ok, uint32_t *q) {
    if (cached) {
      const uint4 w4 = ok && gi < n_grp ? qcache[gi] : make_uint4(0u, 0u, 0u, 0u);
      q[0] = w4.x; q[1] = w4.y; q[2] = w4.z; q[3] = w4.w;
      return;
    }
    const float4 v = load4(L, ok ? gi : n_grp, V, vec_ok);
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) q[c] = (ok && 4 * gi + c < V) ? weight_of(e[c], mx, s) : 0u;
  };
#pragma unroll 1
  for (int c0 = cb; c0 < ce; c0 += SMP_U) {
    uint32_t qq[SMP_U][4];
#pragma unroll
    for (int u = 0; u < SMP_U; ++u) group_q((c0 + u) * 64 + lane, c0 + u < ce, qq[u]);
#pragma unroll
    for (int u = 0; u < SMP_U; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sa += qq[u][c] > tau ? qq[u][c] : 0u;
        sc += qq[u][c] == tau;
      }
  }
  sa = wave_sum_u64(sa);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sc += __shfl_xor(sc, o, 64);
  if (lane == 0) { seg_a[w] = sa; seg_c[w] = sc; }
  __syncthreads();
  uint64_t a0 = 0, t0 = 0;
  int ws = SMP_W - 1;
#pragma unroll 1
  for (int j = 0; j < SMP_W; ++j) {
    const uint64_t a1 = a0 + seg_a[j], t1 = t0 + seg_c[j];
    if (a1 + tau * min(t1, n_tie) > x) { ws = j; break; }
    a0 = a1;
    t0 = t1;
  }
  if (w != ws) return;
  uint64_t cnt = (uint64_t)cb * 256;               // every earlier token runs <= x
  constexpr uint64_t M40 = (1ull << 40) - 1;
#pragma unroll 1
  for (int ch = cb; ch < ce; ++ch) {
    uint32_t qv[4];
    group_q(ch * 64 + lane, true, qv);
    uint64_t la = 0;
    uint32_t lc = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      la += qv[c] > tau ? qv[c] : 0u;
      lc += qv[c] == tau;
    }
    // a chunk's weight above tau is < 2^38 and its tie count <= 256: one
    // 64-bit scan carries both (weight in bits 0..39, count above)
    const uint64_t packed = la | ((uint64_t)lc << 40);
    const uint64_t incl = wave_scan_u64(packed);
    const uint64_t tot = lane63_u64(incl);
    if (a0 + (tot & M40) + tau * min(t0 + (tot >> 40), n_tie) <= x) {
      cnt += 256;
      a0 += tot & M40;
      t0 += tot >> 40;
      continue;
    }
    const uint64_t ex = incl - packed;
    uint64_t a = a0 + (ex & M40), t = t0 + (ex >> 40);
    uint32_t k = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a += qv[c] > tau ? qv[c] : 0u;
      t += qv[c] == tau;
      k += a + tau * min(t, n_tie) <= x;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) k += __shfl_xor(k, o, 64);
    cnt += k;
    break;
  }
  if (lane == 0) out[row] = (int32_t)cnt;
}

}  // namespace

int launch_sample(const float *logits, int64_t ld, int n_rows, int V, const float *temperature,
                  const float *top_p, const uint32_t *uniforms, int32_t *tokens, void *stream) {
  const int vec_ok = (ld % 4 == 0) && (((uintptr_t)logits & 15) == 0);
  const int n_grp = (V + 3) / 4;
  const int cached = n_grp <= SMP_CACHE_GROUPS && temperature != nullptr;
  const size_t lds = cached ? (size_t)n_grp * 16 : 0;
  static bool attr_set = false;  // per process
  if (cached && !attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void *)sample_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             SMP_CACHE_GROUPS * 16);
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  hipLaunchKernelGGL(sample_kernel, dim3(n_rows), dim3(SMP_T), lds, (hipStream_t)stream, logits, ld, V, vec_ok,
                     temperature, top_p, uniforms, tokens, cached);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus
