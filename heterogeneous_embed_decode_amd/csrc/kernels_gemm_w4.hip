// bf16 GEMM on gfx950 matrix cores with one wave per SIMD: C = A B^T for
// the large projections (Efficient Iterative Retrieval with Heterogeneous
// Batching, §3.1: the feed-forward layer runs once over all rows of the
// batch), here the gate/up projection with its SwiGLU epilogue and plain
// bf16 outputs.
//
// Tiling: a 256 x 256 tile of A rows x B rows per workgroup of 4 waves; wave
// (wm, wn) owns a 128 x 128 block as 8 x 8 v_mfma_f32_16x16x32_bf16 blocks
// whose 256 accumulator registers are AGPRs.  K-steps of 32 are fetched by
// buffer loads straight into LDS (a 4-stage ring, 128 KB); per K-step a wave
// reads 16 fragments (0.25 LDS reads per MFMA, a third of the 8-wave
// kernel's 0.75) and issues 8 loads.
//
// The MFMAs are inline asm tied to their accumulators: with the builtin, the
// register allocator copies the 256 accumulators between AGPRs and VGPRs
// inside the loop.  The compiler then does not know these are MFMAs, so it
// cannot insert the wait states an MFMA result needs before another
// instruction reads it, nor the ones a VGPR write needs before an MFMA
// reads it.  Hence the rules this file keeps (a mistake shows up as wrong
// elements 0 and 3 of some MFMA blocks, not as a fault):
//  - one K loop, no tail: K-steps past the end load out-of-range offsets
//    (zeros), so the accumulators keep their registers for the whole loop;
//  - the accumulators are pinned to AGPRs ("+a" asm) after they are zeroed,
//    and after the loop only behind a fence of 48 wait states;
//  - the fragments a step's MFMAs read stay live to the end of the step.
#include "device_common.h"
#include "orthrus_internal.h"

namespace orthrus {

constexpr int W4_BM = 256, W4_BN = 256, W4_BK = 32, W4_S = 4;
constexpr int W4_STAGE = W4_BM * W4_BK;  // bf16 elements per operand per stage (16 KB)
constexpr int W4_LPT = 8;                // loads per lane per K-step (4 A + 4 B)
constexpr uint32_t W4_OOB_ROW = 0x80000000u;  // offset of a row outside the operand
// added to every offset of a K-step past the end; with operands below
// 1 GiB every such offset, and an out-of-range row's, lands at or beyond
// the operand's size, where the buffer unit returns zeros without a
// memory access
constexpr uint32_t W4_PAST_END = 0x40000000u;

typedef __attribute__((address_space(3))) void *lds_ptr_w4;

struct W4Args {
  const uint16_t *A, *B;
  void *C;
  int lda, ldb, ldc, M, N, K, b_up_row;
  uint32_t a_bytes, b_bytes;  // operand sizes for the buffer range check
  float alpha;
};

template <int N>
__device__ __forceinline__ void w4_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// EPI_SWIGLU: the tile's 256 B rows are, per wave column wn, 64 gate rows
// then the 64 up rows of the same output columns, so fragments j and j + 4
// of a wave hold the gate and up values of one output column and the
// output tile is 256 x 128.  EPI_BF16: 256 x 256 outputs, scaled by alpha.
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(W4Args g) {
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_BF16, "SwiGLU or plain bf16 outputs");
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  constexpr int TN = DUAL ? 128 : 256;  // output columns per tile
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *const As = smem;
  uint16_t *const Bs = smem + W4_S * W4_STAGE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile order: groups of 4 tile rows walked column by column; the
  // hardware places workgroup b on XCD b % 8, so each XCD gets a
  // contiguous range of the order and its L2 sees neighbouring tiles
  const int tiles_m = (g.M + W4_BM - 1) / W4_BM, tiles_n = (g.N + TN - 1) / TN, P = tiles_m * tiles_n;
  int t = blockIdx.x;
  {
    const int per = P / 8;
    if (t < per * 8) t = (t % 8) * per + t / 8;
  }
  constexpr int GM = 4;
  const int group = t / (GM * tiles_n), first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM), within = t % (GM * tiles_n);
  const int m0 = (first_m + within % gsz) * W4_BM, n0 = (within / gsz) * TN;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)g.A, (short)0, (int)g.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)g.B, (short)0, (int)g.b_bytes, 0x00020000);
  // Load lanes: instruction i of wave w fills LDS rows (4 i + w) * 16 + lane / 4,
  // 16-byte chunk position lane % 4, with logical chunk (lane % 4) ^ swizzle.
  // A row's chunk swizzle is (row >> 1) & 3.  Measured with
  // SQ_LDS_BANK_CONFLICT on the fragment reads: (row >> 1) & 3 has no bank
  // conflicts, while (row >> 2) & 3, row & 3 and (row ^ (row >> 2)) & 3 are
  // conflicted on half of the LDS-active cycles.
  const int lrow = lane >> 2, pc = lane & 3;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (i * 4 + wave) * 16 + lrow;
    const int kc = pc ^ ((row >> 1) & 3);
    const int gr = m0 + row;
    aoff[i] = gr < g.M ? (uint32_t)(((size_t)gr * g.lda + kc * 8) * 2) : W4_OOB_ROW;
    int br, ncol;
    if (DUAL) {
      const int half = row >> 7, q = row & 127;
      ncol = n0 + half * 64 + (q & 63);
      br = q < 64 ? ncol : g.b_up_row + ncol;
    } else {
      ncol = n0 + row;
      br = ncol;
    }
    boff[i] = ncol < g.N ? (uint32_t)(((size_t)br * g.ldb + kc * 8) * 2) : W4_OOB_ROW;
  }
  const int nk = g.K / W4_BK;
  auto kbytes = [&](int kt) -> uint32_t { return kt < nk ? (uint32_t)(kt * W4_BK * 2) : W4_PAST_END; };
  auto issue_one = [&](uint32_t k2, int st, int idx) {
    if (idx < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_w4)(As + st * W4_STAGE + (idx * 4 + wave) * 512), 16,
                                               aoff[idx] + k2, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_w4)(Bs + st * W4_STAGE + ((idx - 4) * 4 + wave) * 512),
                                               16, boff[idx - 4] + k2, 0, 0, 0);
  };
  // fragment reads: lane l takes row l % 16 of each 16-row block and the 8
  // k of logical chunk l / 16, stored at position (l / 16) ^ ((l >> 1) & 3)
  // (blocks start at multiples of 16 rows, so the swizzle is the lane's own)
  const int fpos = ((lane >> 4) ^ ((lane >> 1) & 3)) * 8 + (lane & 15) * 32;
  const uint16_t *const fa_base = As + wm * 128 * 32 + fpos;
  const uint16_t *const fb_base = Bs + wn * 128 * 32 + fpos;

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i][j]));
    }
  bf16x8_t fa[2][8], fb[2][8];

  // K-step k: 64 MFMAs on the fragments of stage k % 4 (already in
  // registers); after every 4th MFMA one fragment read of step k + 1 from
  // stage (k + 1) % 4, after every 8th one load of step k + 3 into stage
  // (k + 3) % 4.  At the top this wave's loads of steps up to k + 1 have
  // landed (only step k + 2's may be in flight); the barrier makes every
  // wave's visible and retires stage (k - 1) % 4, whose fragments were read
  // during step k - 2 and consumed before the barrier.
  auto step = [&](const int k, auto par_c) {
    constexpr int cu = decltype(par_c)::value, nx = cu ^ 1;
    const int st_n = (k + 1) & 3, st_l = (k + 3) & 3;
    const uint32_t k2 = kbytes(k + 3);
    w4_wait_vmcnt<W4_LPT>();
    __builtin_amdgcn_s_barrier();
    const uint16_t *fan = fa_base + st_n * W4_STAGE, *fbn = fb_base + st_n * W4_STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[cu][j]), "v"(fa[cu][i]));
        const int idx = i * 8 + j;
        if (idx % 4 == 3) {
          const int q = idx / 4;
          if (q < 8) fa[nx][q] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(fan + q * 512));
          else fb[nx][q - 8] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(fbn + (q - 8) * 512));
        }
        if (idx % 8 == 7) issue_one(k2, st_l, idx / 8);
        if (idx % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(fa[cu][i]), "v"(fb[cu][i]));
  };

#pragma unroll
  for (int p = 0; p < W4_S - 1; ++p)
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(kbytes(p), p, q);
  w4_wait_vmcnt<2 * W4_LPT>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 8; ++i) fa[0][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(fa_base + i * 512));
#pragma unroll
  for (int j = 0; j < 8; ++j) fb[0][j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(fb_base + j * 512));
  // pairs of steps; with nk odd the last step multiplies zero-filled stages
  for (int k = 0; k < nk; k += 2) {
    step(k, std::integral_constant<int, 0>{});
    step(k + 1, std::integral_constant<int, 1>{});
  }
  w4_wait_vmcnt<0>();
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));

  // epilogue: the MFMAs take the B fragment as their first operand, so
  // block (i, j) holds C^T: the lane has output row lane % 16 of A block i
  // and the 4 consecutive output columns 4 (lane / 16) .. + 3 of B block j,
  // stored as one 8-byte write where the columns are inside C and aligned
  const int m_l = m0 + wm * 128 + (lane & 15);
  const int c_l = 4 * (lane >> 4);
  const bool vec = (g.ldc & 3) == 0 && ((uintptr_t)g.C & 7) == 0;
  uint16_t *const Cb = (uint16_t *)g.C;
  // v_cvt_pk_bf16_f32: two values to bf16, round to nearest even
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;
  auto cvt2 = [](float lo, float hi) -> uint32_t {
    const bf16x2_v p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
  };
  auto put4 = [&](int m, int n, const float v[4]) {
    if (m >= g.M) return;
    uint16_t *c = Cb + (size_t)m * g.ldc + n;
    uint2 w;
    w.x = cvt2(v[0], v[1]);
    w.y = cvt2(v[2], v[3]);
    if (vec && n + 3 < g.N) {
      *(uint2 *)c = w;
    } else {
      const uint16_t h[4] = {(uint16_t)(w.x & 0xffffu), (uint16_t)(w.x >> 16), (uint16_t)(w.y & 0xffffu),
                             (uint16_t)(w.y >> 16)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < g.N) c[e] = h[e];
    }
  };
  // output values of block row i, column block j: silu(g) u = g u / (1 +
  // 2^(-g log2 e)) of the gate (j) and up (j + 4) blocks, or alpha acc
  auto value4 = [&](int i, int j, float o[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (DUAL) {
        const float gt = acc[i][j][e], up = acc[i][j + 4][e];
        const float den = 1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f);
        o[e] = gt * up * __builtin_amdgcn_rcpf(den);
      } else {
        o[e] = g.alpha * acc[i][j][e];
      }
    }
  };
  constexpr int NJ = DUAL ? 4 : 8;
  const int nw = n0 + wn * (TN / 2) + c_l;
  if (vec && m0 + W4_BM <= g.M && n0 + TN <= g.N) {
    // the whole tile is inside C: no per-element checks, so the scheduler
    // can overlap the blocks' arithmetic
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t *const crow = Cb + (size_t)(m_l + i * 16) * g.ldc + nw;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float o[4];
        value4(i, j, o);
        uint2 w;
        w.x = cvt2(o[0], o[1]);
        w.y = cvt2(o[2], o[3]);
        *(uint2 *)(crow + j * 16) = w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float o[4];
        value4(i, j, o);
        put4(m_l + i * 16, nw + j * 16, o);
      }
  }
}

template <int EPI>
static int launch_w4(const W4Args &a, hipStream_t s) {
  constexpr int TN = EPI == EPI_SWIGLU ? 128 : 256;
  const int tiles = ((a.M + W4_BM - 1) / W4_BM) * ((a.N + TN - 1) / TN);
  if (tiles == 0) return 0;
  constexpr int lds = 2 * W4_S * W4_STAGE * (int)sizeof(uint16_t);
  auto kern = gemm_w4_kernel<EPI>;
  static bool attr_set = false;  // per process; the library drives one device at a time
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(tiles), dim3(256), lds, s, a);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

bool gemm_w4_eligible(int lda, int ldb, int M, int N, int K, int epi, int b_up_row) {
  if (epi != EPI_SWIGLU && epi != EPI_BF16) return false;
  if (M < 256 || N < 256 || K < W4_BK || K % W4_BK != 0 || lda % 8 != 0 || ldb % 8 != 0) return false;
  const size_t a_bytes = (size_t)M * lda * 2;
  const size_t b_rows = epi == EPI_SWIGLU ? (size_t)b_up_row + N : (size_t)N;
  const size_t b_bytes = b_rows * ldb * 2;
  return a_bytes < (size_t(1) << 30) && b_bytes < (size_t(1) << 30);
}

int launch_gemm_w4(const uint16_t *A, int lda, const uint16_t *B, int ldb, void *C, int ldc, int M, int N, int K,
                   int epi, int b_up_row, float alpha, void *stream) {
  if (!gemm_w4_eligible(lda, ldb, M, N, K, epi, b_up_row)) return (int)hipErrorInvalidValue;
  W4Args a{};
  a.A = A; a.B = B; a.C = C;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc; a.M = M; a.N = N; a.K = K; a.b_up_row = b_up_row;
  a.a_bytes = (uint32_t)((size_t)M * lda * 2);
  a.b_bytes = (uint32_t)(((epi == EPI_SWIGLU ? (size_t)b_up_row : 0) + N) * ldb * 2);
  a.alpha = alpha;
  hipStream_t s = (hipStream_t)stream;
  return epi == EPI_SWIGLU ? launch_w4<EPI_SWIGLU>(a, s) : launch_w4<EPI_BF16>(a, s);
}

}  // namespace orthrus
