// bf16 GEMM on gfx950 matrix cores: C = A B^T, fp32 accumulation.
//
// Serves every projection of the decoder layer (Efficient Iterative
// Retrieval with Heterogeneous Batching, §3.1: the attention and
// feed-forward layers are applied once to all rows of the batch) and the
// LM head.  Epilogues fuse what follows each projection: bf16 store (QKV),
// fp32 residual add (output and down projections), SwiGLU of paired
// gate/up columns, fp32 store (logits).  The embedding adapter (§2.2
// Parameter sharing) is applied as extra K-steps over [U | B_lora] for
// rows below the embedding-row count, so generation rows never see it.
//
// Tiling: BM x BN output tile per workgroup of WM x WN waves, K-steps of
// 64 staged through LDS with an XOR swizzle of 16-byte chunks, double
// buffered; each wave issues v_mfma_f32_32x32x16_bf16 on 32x32 blocks.
#include "device_common.h"
#include "orthrus_internal.h"

namespace orthrus {

struct GemmArgs {
  const uint16_t *A;
  const uint16_t *B;
  void *C;
  int lda, ldb, ldc, M, N, K, b_up_row;
  float alpha;
  // adapter extension (rows < lrows)
  const uint16_t *U;
  const uint16_t *Bx;
  int ldu, r, lrows, sec1, sec2;
};

constexpr int BK = 64;

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM *WN * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NT = WM * WN * 64;
  constexpr int BNB = DUAL ? 2 * BN : BN;      // B rows staged per tile
  constexpr int WTM = BM / WM;                  // wave tile rows
  constexpr int WCN = BN / WN;                  // wave tile output columns
  constexpr int MI = WTM / 32;
  constexpr int NI = DUAL ? 2 * (WCN / 32) : WCN / 32;
  constexpr int A_LD = BM * (BK / 8) / NT;
  constexpr int B_LD = BNB * (BK / 8) / NT;
  static_assert(A_LD * NT == BM * BK / 8 && B_LD * NT == BNB * BK / 8, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BNB * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // tile order: XCD-contiguous ranges, then groups of GM tile rows walked
  // column by column so that resident workgroups share B tiles in L2
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int P = tiles_m * tiles_n;
  int pid = blockIdx.x;
  {
    const int per = P / 8;
    if (pid < per * 8) pid = (pid % 8) * per + pid / 8;
  }
  constexpr int GM = 16;
  const int group = pid / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int within = pid % (GM * tiles_n);
  const int tm = first_m + within % gsz;
  const int tn = within / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  // B tile row rr -> output column of that row and its global B row
  auto b_src_row = [&](int rr, int &ncol) -> int {
    if (DUAL) {
      const int c = rr < BN ? rr : rr - BN;
      ncol = n0 + c;
      return rr < BN ? ncol : g.b_up_row + ncol;
    }
    ncol = n0 + rr;
    return ncol;
  };

  // phase 0: main operands over K; phase 1: adapter operands over ldu
  auto run_phase = [&](const int phase, const int Kp) {
    u32x4_t ra[A_LD], rb[B_LD];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int c = tid + i * NT;
        const int row = c / (BK / 8), kc = c % (BK / 8);
        const int gr = m0 + row, k = k0 + kc * 8;
        if (phase == 0)
          ra[i] = (gr < g.M && k < Kp) ? *(const u32x4_t *)(g.A + (size_t)gr * g.lda + k) : zero4;
        else
          ra[i] = (gr < g.lrows && gr < g.M && k < Kp) ? *(const u32x4_t *)(g.U + (size_t)gr * g.ldu + k)
                                                         : zero4;
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int c = tid + i * NT;
        const int rr = c / (BK / 8), kc = c % (BK / 8);
        const int k = k0 + kc * 8;
        int ncol;
        const int br = b_src_row(rr, ncol);
        if (phase == 0) {
          rb[i] = (ncol < g.N && k < Kp) ? *(const u32x4_t *)(g.B + (size_t)br * g.ldb + k) : zero4;
        } else {
          const int sec = ncol < g.sec1 ? 0 : (ncol < g.sec2 ? 1 : 2);
          const bool ok = ncol < g.N && k < Kp && (k / g.r) == sec;
          rb[i] = ok ? *(const u32x4_t *)(g.Bx + (size_t)ncol * g.r + (k % g.r)) : zero4;
        }
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int c = tid + i * NT;
        const int row = c / (BK / 8), kc = c % (BK / 8);
        *(u32x4_t *)(&As[buf][row * BK + ((kc ^ (row & 7)) * 8)]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int c = tid + i * NT;
        const int rr = c / (BK / 8), kc = c % (BK / 8);
        *(u32x4_t *)(&Bs[buf][rr * BK + ((kc ^ (rr & 7)) * 8)]) = rb[i];
      }
    };
    const int nk = (Kp + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int chunk = kk * 2 + (lane >> 5);
        bf16x8_t a[MI], b[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int row = wm * WTM + i * 32 + (lane & 31);
          a[i] = __builtin_bit_cast(bf16x8_t,
                                    *(const u32x4_t *)(&As[cur][row * BK + ((chunk ^ (row & 7)) * 8)]));
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          int rr;
          if (DUAL)
            rr = (j < NI / 2 ? 0 : BN) + wn * WCN + (j % (NI / 2)) * 32 + (lane & 31);
          else
            rr = wn * WCN + j * 32 + (lane & 31);
          b[j] = __builtin_bit_cast(bf16x8_t,
                                    *(const u32x4_t *)(&Bs[cur][rr * BK + ((chunk ^ (rr & 7)) * 8)]));
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }
  };

  run_phase(0, g.K);
  if (!DUAL && g.U != nullptr && m0 < g.lrows) run_phase(1, g.ldu);

  // epilogue: lane holds column (lane & 31) and rows 8*(e/4) + 4*(lane/32) + e%4
  const int jc = lane & 31;
  const int rbase = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    if (DUAL) {
#pragma unroll
      for (int j = 0; j < NI / 2; ++j) {
        const int n = n0 + wn * WCN + j * 32 + jc;
        if (n >= g.N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WTM + i * 32 + (e / 4) * 8 + rbase + (e % 4);
          if (m >= g.M) continue;
          const float gt = acc[i][j][e], up = acc[i][j + NI / 2][e];
          const float s = gt / (1.f + expf(-gt));
          ((uint16_t *)g.C)[(size_t)m * g.ldc + n] = (uint16_t)f2bf(s * up);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = n0 + wn * WCN + j * 32 + jc;
        if (n >= g.N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * WTM + i * 32 + (e / 4) * 8 + rbase + (e % 4);
          if (m >= g.M) continue;
          const size_t o = (size_t)m * g.ldc + n;
          const float v = acc[i][j][e];
          if (EPI == EPI_BF16) ((uint16_t *)g.C)[o] = (uint16_t)f2bf(g.alpha * v);
          else if (EPI == EPI_F32) ((float *)g.C)[o] = g.alpha * v;
          else ((float *)g.C)[o] += v;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
static int launch_cfg(const GemmArgs &a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return 0;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, EPI>), dim3(tiles), dim3(WM * WN * 64), 0, s, a);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_gemm(const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc, int M,
                int N, int K, int epi, int b_up_row, float alpha, const LoraArgs *lora,
                void *stream) {
  if (M <= 0 || N <= 0) return 0;
  GemmArgs a{};
  a.A = A; a.B = B; a.C = C;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc; a.M = M; a.N = N; a.K = K; a.b_up_row = b_up_row;
  a.alpha = alpha;
  if (lora && lora->U && lora->rows > 0 && lora->r > 0) {
    a.U = lora->U; a.Bx = lora->Bx; a.ldu = lora->ldu; a.r = lora->r; a.lrows = lora->rows;
    a.sec1 = lora->sec1; a.sec2 = lora->sec2;
  }
  hipStream_t s = (hipStream_t)stream;
  switch (epi) {
    case EPI_BF16: return launch_cfg<128, 128, 2, 2, EPI_BF16>(a, s);
    case EPI_F32: return launch_cfg<128, 128, 2, 2, EPI_F32>(a, s);
    case EPI_RESID: return launch_cfg<128, 128, 2, 2, EPI_RESID>(a, s);
    case EPI_SWIGLU: return launch_cfg<128, 64, 2, 2, EPI_SWIGLU>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace orthrus
