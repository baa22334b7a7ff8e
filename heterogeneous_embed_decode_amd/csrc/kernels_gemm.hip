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
// BK fetched by buffer loads straight into LDS (XOR swizzle of 16-byte
// chunks, an S-stage ring), each wave issuing v_mfma_f32_32x32x16_bf16 on
// 32x32 blocks.  Operands must be smaller than 2 GiB (32-bit buffer offsets).
#include "device_common.h"
#include "orthrus_internal.h"

#include <type_traits>

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
  // residual epilogue only: 0 = one workgroup per output tile; otherwise
  // the grid size, whole tiles first and the rest as stream-K slices
  int sk_grid;
  int group_m;  // tile rows per group of the tile order (0 = default)
  // QKV epilogue only (head dim 128)
  const float *rope_cs;
  const int32_t *slot;
  uint16_t *kc, *vc;
  int q_cols, kv_cols, n_kv, ps;
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// MFMA block size: 32 selects v_mfma_f32_32x32x16_bf16, 16 selects
// v_mfma_f32_16x16x32_bf16.  Both have the same peak rate.  In a
// register-only MFMA loop on MI355X with random bf16 operands the 16x16 form
// sustained 80-82 % of the bf16 peak against 65-73 % for the 32x32 form
// (with zero operands both reach about 98 %: the chip is power-limited),
// but in this kernel both forms ran within 1 % of each other, and the 16x16
// form needs more registers for its 32-deep fragments, so 32 is used.
constexpr int MT = 32;

// LDS swizzle of the 16-byte chunks of one tile row (BK/8 chunks).
// ds_read_b128 is served 16 lanes at a time across 64 banks (256 bytes);
// the 16 rows a half-wave reads must land on 16 distinct 16-byte bank
// slots.  A 128-byte row (BK = 64) has 8 chunks, so the chunk is XORed
// with bits 1..3 of the row; a 64-byte row (BK = 32) has 4 chunks, XORed
// with bits 2..3.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `tiles_after` tiles of LPT loads per lane are in flight
template <int LPT, int S>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  if (S >= 5 && tiles_after >= 3) wait_vmcnt<(S >= 5 ? 3 : 0) * LPT>();
  else if (S >= 4 && tiles_after >= 2) wait_vmcnt<(S >= 4 ? 2 : 0) * LPT>();
  else if (S >= 3 && tiles_after >= 1) wait_vmcnt<(S >= 3 ? 1 : 0) * LPT>();
  else wait_vmcnt<0>();
}

template <int BM, int BN, int WM, int WN, int BK, int S, int EPI>
__global__ __launch_bounds__(WM *WN * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int BNB = DUAL ? 2 * BN : BN;      // B rows staged per tile
  constexpr int WTM = BM / WM;                  // wave tile rows
  constexpr int WCN = BN / WN;                  // wave tile output columns
  constexpr int MI = WTM / MT;                  // MFMA blocks per wave tile
  constexpr int NI = DUAL ? 2 * (WCN / MT) : WCN / MT;
  constexpr int KS = MT == 32 ? 16 : 32;        // k per MFMA
  constexpr int NE = MT == 32 ? 16 : 4;         // accumulators per lane per block
  using acc_t = typename std::conditional<MT == 32, f32x16_t, f32x4_t>::type;
  constexpr int CPR = BK / 8;                   // 16-byte chunks per tile row
  constexpr int RPI = 64 / CPR;                 // tile rows per wave load instruction
  constexpr int A_ROUNDS = BM / (RPI * NW);
  constexpr int B_ROUNDS = BNB / (RPI * NW);
  constexpr int LPT = A_ROUNDS + B_ROUNDS;      // loads per lane per tile
  static_assert(A_ROUNDS * RPI * NW == BM && B_ROUNDS * RPI * NW == BNB, "tile/threads mismatch");
  static_assert(S >= 2 && S <= 5, "2..5 stages");

  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *const As0 = smem;                   // [S][BM * BK]
  uint16_t *const Bs0 = smem + S * BM * BK;     // [S][BNB * BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // tile order: groups of GM tile rows walked column by column, so the ~32
  // workgroups resident on one XCD cover about 4 x 8 tiles and share both
  // A and B tiles in that XCD's L2 (measured best at GM = 4)
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int P = tiles_m * tiles_n;
  const int GM = g.group_m > 0 ? g.group_m : 4;
  int m0 = 0, n0 = 0;
  auto set_tile = [&](int t) {
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int within = t % (GM * tiles_n);
    m0 = (first_m + within % gsz) * BM;
    n0 = (within / gsz) * BN;
  };
  // hardware places workgroup b on XCD b % 8: give each XCD a contiguous
  // range of logical indices so its L2 sees neighbouring tiles
  auto xcd_remap = [](int b, int n) {
    const int per = n / 8;
    return b < per * 8 ? (b % 8) * per + b / 8 : b;
  };

  acc_t acc[MI][NI];

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

  // Operand tiles are fetched with buffer loads that write straight into
  // LDS (16 bytes per lane, lane t of a wave at M0 + 16 t).  The XOR swizzle
  // is applied on the global side: the lane that fills LDS chunk (row, pc)
  // fetches logical chunk pc ^ swz(row).  Rows or K-chunks outside the
  // operand get an out-of-range offset, which the buffer unit returns as
  // zeros, so the loop has no branches.
  constexpr uint32_t OOB = 0x80000000u;
  const int lrow = lane / CPR, pc = lane % CPR;

  // MFMA operand fragments of one KS-wide k slice: lane l holds row (or
  // column) l % MT and the 8 consecutive k of chunk l / MT of the slice
  auto load_frags = [&](const uint16_t *As, const uint16_t *Bs, int kk, bf16x8_t *a, bf16x8_t *b) {
    const int chunk = kk * (KS / 8) + lane / MT;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = wm * WTM + i * MT + (lane & (MT - 1));
      a[i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(&As[row * BK + ((chunk ^ swz<BK>(row)) * 8)]));
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      int rr;
      if (DUAL)
        rr = (j < NI / 2 ? 0 : BN) + wn * WCN + (j % (NI / 2)) * MT + (lane & (MT - 1));
      else
        rr = wn * WCN + j * MT + (lane & (MT - 1));
      b[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(&Bs[rr * BK + ((chunk ^ swz<BK>(rr)) * 8)]));
    }
  };
  // all k slices of one stage; fragments of slice k+1 are read before the
  // MFMAs of slice k are issued so LDS latency hides behind matrix work.
  // `loads` issues the global loads of a later K-step; they are placed one
  // after each of the first MFMAs of slice 0, so the waves of a SIMD, which
  // leave the step's barrier together, keep the matrix pipe busy while the
  // loads go out.
  auto compute = [&](int st, auto &&loads) {
    const uint16_t *As = As0 + st * BM * BK, *Bs = Bs0 + st * BNB * BK;
    bf16x8_t a[2][MI], b[2][NI];
    load_frags(As, Bs, 0, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < BK / KS; ++kk) {
      if (kk + 1 < BK / KS) load_frags(As, Bs, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if constexpr (MT == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
        }
      if (kk == 0) {
        loads();
#pragma unroll
        for (int q = 0; q < LPT; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one VMEM
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // phase 0: main operands over K; phase 1: adapter operands over ldu
  auto run_phase = [&](const int phase, const int Kp, const int kb, const int ke) {
    const uint16_t *abase = phase == 0 ? g.A : g.U;
    const int alda = phase == 0 ? g.lda : g.ldu;
    const int arows = phase == 0 ? g.M : min(g.M, g.lrows);
    const uint16_t *bbase = phase == 0 ? g.B : g.Bx;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)abase, (short)0, (int)0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)bbase, (short)0, (int)0x7fffffff, 0x00020000);
    // per-lane byte offsets at k0 = 0 (OOB when the row is outside)
    uint32_t aoff[A_ROUNDS], boff[B_ROUNDS];
    int akc[A_ROUNDS], bkc[B_ROUNDS];
#pragma unroll
    for (int i = 0; i < A_ROUNDS; ++i) {
      const int row = (i * NW + wave) * RPI + lrow;
      const int kc = pc ^ swz<BK>(row);
      const int gr = m0 + row;
      akc[i] = kc * 8;
      aoff[i] = gr < arows ? (uint32_t)(((size_t)gr * alda + kc * 8) * 2) : OOB;
    }
#pragma unroll
    for (int i = 0; i < B_ROUNDS; ++i) {
      const int rr = (i * NW + wave) * RPI + lrow;
      const int kc = pc ^ swz<BK>(rr);
      int ncol;
      const int br = b_src_row(rr, ncol);
      if (phase == 0) {
        bkc[i] = kc * 8;
        boff[i] = ncol < g.N ? (uint32_t)(((size_t)br * g.ldb + kc * 8) * 2) : OOB;
      } else {
        // adapter expand: column ncol holds s*B for its own section only;
        // element k of the extension is B[ncol][k - sec*r] when that is in [0, r)
        const int sec = ncol < g.sec1 ? 0 : (ncol < g.sec2 ? 1 : 2);
        bkc[i] = kc * 8 - sec * g.r;
        boff[i] = ncol < g.N ? (uint32_t)(((size_t)ncol * g.r + kc * 8 - sec * g.r) * 2) : OOB;
      }
    }
    // FULL: all BK columns of the step lie inside the main operands, so
    // only the row check (already folded into the offset) remains
    auto issue = [&](int kt, auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const int k0 = kt * BK, st = kt % S;
#pragma unroll
      for (int i = 0; i < A_ROUNDS; ++i) {
        uint32_t off;
        if (FULL) {
          off = aoff[i] + (uint32_t)(k0 * 2);  // OOB + k0*2 stays out of range
        } else {
          const bool ok = (k0 + akc[i]) < Kp && aoff[i] != OOB;
          off = ok ? aoff[i] + (uint32_t)(k0 * 2) : OOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_ptr_t)(As0 + st * BM * BK + (i * NW + wave) * 512), 16, off, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < B_ROUNDS; ++i) {
        uint32_t off;
        if (FULL && phase == 0) {
          off = boff[i] + (uint32_t)(k0 * 2);
        } else {
          bool ok = boff[i] != OOB;
          if (phase == 0) ok = ok && (k0 + bkc[i]) < Kp;
          else ok = ok && (k0 + bkc[i]) >= 0 && (k0 + bkc[i]) < g.r;
          off = ok ? boff[i] + (uint32_t)(k0 * 2) : OOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_ptr_t)(Bs0 + st * BNB * BK + (i * NW + wave) * 512), 16, off, 0, 0, 0);
      }
    };
    // S-stage ring over K-steps [kb, ke): steps kt+1 .. kt+S-2 stay in
    // flight while step kt is consumed; one barrier per step both publishes
    // step kt and retires the stage that the next issue overwrites.  The
    // bare s_barrier avoids the fence of __syncthreads, which would drain
    // the loads in flight.  The loop is split so that each part is one
    // straight-line block (the loads can then be scheduled among the
    // MFMAs): steps that load a full K-step, steps that load a ragged or
    // adapter step, and the last S-1 steps, which load nothing.
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
      if (kb + p < ke) issue(kb + p, std::false_type{});
    const int nfull = phase == 0 ? Kp / BK : 0;
    int kt = kb;
    for (; kt + S - 1 < ke && kt + S - 1 < nfull; ++kt) {
      wait_tiles<LPT, S>(S - 2);
      __builtin_amdgcn_s_barrier();
      compute(kt % S, [&] { issue(kt + S - 1, std::true_type{}); });
    }
    for (; kt + S - 1 < ke; ++kt) {
      wait_tiles<LPT, S>(S - 2);
      __builtin_amdgcn_s_barrier();
      compute(kt % S, [&] { issue(kt + S - 1, std::false_type{}); });
    }
    for (; kt < ke; ++kt) {
      wait_tiles<LPT, S>(min(S - 2, ke - 1 - kt));
      __builtin_amdgcn_s_barrier();
      compute(kt % S, [] {});
    }
  };

  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[i][j][e] = 0.f;
  };

  const int nk = (g.K + BK - 1) / BK;
  const bool lora_tile_possible = !DUAL && g.U != nullptr;
  // epilogue: in each MT x MT block the lane holds column lane % MT and
  // rows erow(e): 8*(e/4) + 4*(lane/32) + e%4 for MT = 32, 4*(lane/16) + e
  // for MT = 16 (rows e and e+1 are adjacent for even e in both)
  // residual: hardware float atomic add into x (no return value to wait
  // for); stream-K partial sums of one tile land in no fixed order
  // bf16 outputs: two rows (e, e+1) of the lane's column are converted by
  // one v_cvt_pk_bf16_f32 and stored as the low and high halves
  auto store_bf16_pair = [&](int m, int n, float v0, float v1) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;
    const bf16x2_v pk = {(__bf16)v0, (__bf16)v1};
    const uint32_t w = __builtin_bit_cast(uint32_t, pk);
    uint16_t *c = (uint16_t *)g.C + (size_t)m * g.ldc + n;
    if (m < g.M) c[0] = (uint16_t)(w & 0xffffu);
    if (m + 1 < g.M) c[g.ldc] = (uint16_t)(w >> 16);
  };
  // whole: this workgroup ran every K-step of the tile, so a residual
  // output is a plain read-modify-write of x (its loads batched per 32-row
  // block); stream-K slices of a tile add theirs with float atomics
  auto epilogue = [&](const bool whole) {
    const int jc = lane & (MT - 1);
    auto erow = [&](int e) { return MT == 32 ? (e / 4) * 8 + (lane >> 5) * 4 + (e % 4) : (lane >> 4) * 4 + e; };
    const int mw = m0 + wm * WTM, nw = n0 + wn * WCN;
    if (EPI == EPI_RESID && whole) {
      // 32-bit buffer offsets; rows past M or columns past N get an
      // out-of-range offset, which loads as zero and is not stored.  The
      // lane's values are taken in groups of 16; the x values of the next
      // group are loaded before the current group is stored.
      const __amdgpu_buffer_rsrc_t rx =
          __builtin_amdgcn_make_buffer_rsrc(g.C, (short)0, (int)0x7fffffff, 0x00020000);
      constexpr int NV = MI * NI * NE, NG = NV / 16;
      static_assert(NV % 16 == 0, "whole groups of 16 values");
      auto xoff = [&](int v) -> uint32_t {
        const int blk = v / NE, e = v % NE;
        const int n = nw + (blk % NI) * MT + jc;
        const int m = mw + (blk / NI) * MT + erow(e);
        return (m < g.M && n < g.N) ? (uint32_t)((m * g.ldc + n) * 4) : OOB;
      };
      uint32_t xv[2][16];
#pragma unroll
      for (int u = 0; u < 16; ++u) xv[0][u] = __builtin_amdgcn_raw_buffer_load_b32(rx, xoff(u), 0, 0);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (gi + 1 < NG) {
#pragma unroll
          for (int u = 0; u < 16; ++u)
            xv[(gi + 1) & 1][u] = __builtin_amdgcn_raw_buffer_load_b32(rx, xoff((gi + 1) * 16 + u), 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int v = gi * 16 + u, blk = v / NE;
          const float r = __uint_as_float(xv[gi & 1][u]) + acc[blk / NI][blk % NI][v % NE];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(r), rx, xoff(v), 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (DUAL) {
        // silu(g) u = g u / (1 + 2^(-g log2 e)): v_exp_f32 and v_rcp_f32
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) {
          const int n = nw + j * MT + jc;
          if (n >= g.N) continue;
#pragma unroll
          for (int e = 0; e < NE; e += 2) {
            const int m = mw + i * MT + erow(e);
            float o2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float gt = acc[i][j][e + u], up = acc[i][j + NI / 2][e + u];
              const float den = 1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f);
              o2[u] = gt * up * __builtin_amdgcn_rcpf(den);
            }
            store_bf16_pair(m, n, o2[0], o2[1]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int n = nw + j * MT + jc;
          if (n >= g.N) continue;
          if (EPI == EPI_BF16) {
#pragma unroll
            for (int e = 0; e < NE; e += 2) {
              const int m = mw + i * MT + erow(e);
              store_bf16_pair(m, n, g.alpha * acc[i][j][e], g.alpha * acc[i][j][e + 1]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              const int m = mw + i * MT + erow(e);
              if (m >= g.M) continue;
              const size_t o = (size_t)m * g.ldc + n;
              const float v = acc[i][j][e];
              if (EPI == EPI_F32) ((float *)g.C)[o] = g.alpha * v;
              else unsafeAtomicAdd((float *)g.C + o, v);  // stream-K slice: x += v
            }
          }
        }
      }
    }
  };

  // QKV epilogue (Efficient Iterative Retrieval with Heterogeneous
  // Batching, §3.1: every row of the batch goes through the same projection;
  // its keys and values enter the paged cache).  A 256-column tile holds two
  // whole heads of one section (q, k or v; head dim 128).  The rotate-half
  // partner of dim i < 64 is dim i + 64, which sits in another wave's
  // accumulators, so the tile goes through LDS in fp32, 128 rows at a time
  // ([row][col], col XOR 32 on rows with bit 2 set: the two 32-lane halves
  // of a store land on different banks, and a 16-lane read of 64
  // consecutive columns stays conflict-free).  Then thread t (of 512)
  // rotates 4 pairs (dims 4 (t % 16) .. +3 and their partners) of both
  // heads on rows t / 16 + 32 k: out_a = a cos - b sin, out_b = b cos + a sin,
  // one rounding to bf16, and stores 8 bytes per half head, 16 lanes per
  // 128-byte run: q into qkv, k and v into the row's KV page slot.  The
  // rows' cos/sin and KV slots are loaded before the LDS exchange that
  // precedes their use, so their latency overlaps it.
  auto qkv_epilogue = [&]() {
    static_assert(EPI != EPI_QKV || (BM == 256 && BN == 256 && WM == 2 && WN == 4 && MT == 32),
                  "the QKV epilogue assumes 256x256 tiles on 2x4 waves");
    constexpr int RP = NT / 16;   // rows covered by one pass of all threads
    constexpr int NR = 128 / RP;  // rows per thread per half tile
    static_assert(EPI != EPI_QKV || NR * RP == 128, "whole row passes");
    float *xs = (float *)smem;  // 128 x 256 fp32 = the 128 KB of the two stages
    const int sec = n0 < g.q_cols ? 0 : (n0 < g.q_cols + g.kv_cols ? 1 : 2);
    const int jc = lane & (MT - 1);
    const int g4 = tid & 15;
    uint16_t *const dst0 = sec == 0 ? (uint16_t *)g.C : (sec == 1 ? g.kc : g.vc);
    const int kvh0 = sec == 0 ? 0 : (n0 - g.q_cols - (sec == 2 ? g.kv_cols : 0)) / 128;
    const size_t head_stride = sec == 0 ? 128 : (size_t)g.ps * 128;
    float4 cpre[NR] = {}, spre[NR] = {};
    int spre_slot[NR] = {};
    auto prefetch = [&](int half) {
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const int m = min(m0 + half * 128 + (tid >> 4) + RP * it, g.M - 1);
        if (sec < 2) {
          cpre[it] = *(const float4 *)(g.rope_cs + (size_t)m * 128 + g4 * 4);
          spre[it] = *(const float4 *)(g.rope_cs + (size_t)m * 128 + 64 + g4 * 4);
        }
        if (sec > 0) spre_slot[it] = g.slot[m];
      }
    };
    prefetch(0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // the stages (or the previous half) are no longer read
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < NE; ++e) {
              const int row = i * MT + (e / 4) * 8 + (lane >> 5) * 4 + (e % 4);
              const int col = wn * WCN + j * MT + jc;
              xs[row * 256 + (col ^ (((row >> 2) & 1) << 5))] = g.alpha * acc[i][j][e];
            }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const int r = (tid >> 4) + RP * it;
        const int m = m0 + half * 128 + r;
        const int sw = ((r >> 2) & 1) << 5;
        size_t rowbase;  // element offset of the row's first head in the tile
        if (sec == 0) {
          rowbase = (size_t)m * g.ldc + n0;
        } else {
          const int sl = spre_slot[it];
          const int page = sl / g.ps, off = sl - page * g.ps;
          rowbase = (((size_t)page * g.n_kv + kvh0) * g.ps + off) * 128;
        }
        const float cc[4] = {cpre[it].x, cpre[it].y, cpre[it].z, cpre[it].w};
        const float ss[4] = {spre[it].x, spre[it].y, spre[it].z, spre[it].w};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ca = hh * 128 + g4 * 4;
          const float4 a = *(const float4 *)&xs[r * 256 + (ca ^ sw)];
          const float4 b = *(const float4 *)&xs[r * 256 + ((ca + 64) ^ sw)];
          const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
          float oa[4], ob[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            oa[u] = sec < 2 ? av[u] * cc[u] - bv[u] * ss[u] : av[u];
            ob[u] = sec < 2 ? bv[u] * cc[u] + av[u] * ss[u] : bv[u];
          }
          if (m < g.M) {
            uint16_t *dst = dst0 + rowbase + hh * head_stride + g4 * 4;
            uint2 wa, wb;
            wa.x = pack_bf2(oa[0], oa[1]); wa.y = pack_bf2(oa[2], oa[3]);
            wb.x = pack_bf2(ob[0], ob[1]); wb.y = pack_bf2(ob[2], ob[3]);
            *(uint2 *)dst = wa;
            *(uint2 *)(dst + 64) = wb;
          }
        }
      }
      if (half == 0) prefetch(1);
    }
  };

  if (g.sk_grid == 0 && gridDim.y > 1) {
    // K split over gridDim.y (fp32 outputs only): split y runs K-steps
    // [nk y / ny, nk (y + 1) / ny) of its tile and stores its partial sums
    // in slab y of C, [y][M][ldc]; the caller adds the slabs in order
    if constexpr (EPI == EPI_F32) {
      set_tile(xcd_remap(blockIdx.x, P));
      zero_acc();
      const int ny = gridDim.y, y = blockIdx.y;
      g.C = (float *)g.C + (size_t)y * g.M * g.ldc;
      run_phase(0, g.K, (int)((long)nk * y / ny), (int)((long)nk * (y + 1) / ny));
      epilogue(true);
    }
  } else if (g.sk_grid == 0) {
    set_tile(xcd_remap(blockIdx.x, P));
    zero_acc();
    run_phase(0, g.K, 0, nk);
    if (lora_tile_possible && m0 < g.lrows) {
      __builtin_amdgcn_s_barrier();  // all waves are done with the last stage
      run_phase(1, g.ldu, 0, (g.ldu + BK - 1) / BK);
    }
    if constexpr (EPI == EPI_QKV) qkv_epilogue();
    else epilogue(true);
  } else if (EPI == EPI_RESID) {
    // residual projections on a grid of sk_grid workgroups (one per CU):
    // whole tiles first, in rounds of sk_grid consecutive tiles of the
    // grouped order (so the tiles in flight at once are neighbours), then
    // the tiles left over shared out as equal slices of their K-steps
    // (stream-K)
    const int w = xcd_remap(blockIdx.x, g.sk_grid);
    const int q = P / g.sk_grid;
    const int P_dp = q * g.sk_grid;
    for (int t = w; t < P_dp; t += g.sk_grid) {
      set_tile(t);
      zero_acc();
      __builtin_amdgcn_s_barrier();  // the previous tile's stages are retired
      run_phase(0, g.K, 0, nk);
      if (lora_tile_possible && m0 < g.lrows) {
        __builtin_amdgcn_s_barrier();
        run_phase(1, g.ldu, 0, (g.ldu + BK - 1) / BK);
      }
      epilogue(true);
    }
    const long total = (long)(P - P_dp) * nk;
    long it = total * w / g.sk_grid;
    const long it_end = total * (w + 1) / g.sk_grid;
    while (it < it_end) {
      const int t = (int)(it / nk);
      const int kb = (int)(it % nk);
      const int ke = (int)min((long)nk, kb + (it_end - it));
      set_tile(P_dp + t);
      zero_acc();
      __builtin_amdgcn_s_barrier();  // previous segment's stages are retired
      run_phase(0, g.K, kb, ke);
      if (ke == nk && lora_tile_possible && m0 < g.lrows) {
        __builtin_amdgcn_s_barrier();
        run_phase(1, g.ldu, 0, (g.ldu + BK - 1) / BK);
      }
      epilogue(kb == 0 && ke == nk);
      it += ke - kb;
    }
  }
}

template <int BM, int BN, int WM, int WN, int BK, int S, int EPI>
static int launch_cfg(GemmArgs a, hipStream_t s, int sk_grid = 0, int k_splits = 1) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (tiles == 0) return 0;
  constexpr int BNB = (EPI == EPI_SWIGLU) ? 2 * BN : BN;
  constexpr size_t lds = (size_t)S * (BM + BNB) * BK * sizeof(uint16_t);
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, BK, S, EPI>;
  static bool attr_set = false;  // per process; the library drives one device at a time
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  a.sk_grid = sk_grid;
  hipLaunchKernelGGL(kern, dim3(sk_grid > 0 ? sk_grid : tiles, k_splits), dim3(WM * WN * 64), lds, s, a);
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int gemm_cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
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
  // Tile shapes measured on MI355X for the decoder's projections: 256-row
  // tiles on 8 waves (two per SIMD) for large problems; a 64-row tile with a
  // 4-deep load ring for few rows (LM head, decode-only batches), where the
  // weights stream from HBM; 128x128 on 4 waves otherwise.
  const bool big = M >= 512 && N >= 1024;
  const bool skinny = M <= 64;
  const bool no_adapter = a.U == nullptr;
  switch (epi) {
    case EPI_BF16:
      if (big && no_adapter && gemm_w4_eligible(lda, ldb, M, N, K, EPI_BF16, 0))
        return launch_gemm_w4(A, lda, B, ldb, C, ldc, M, N, K, EPI_BF16, 0, alpha, stream);
      if (big) return launch_cfg<256, 256, 2, 4, 64, 2, EPI_BF16>(a, s);
      // few output columns (the adapter shrink, N = 3 x rank): small tiles
      // so that more workgroups share the long K loop
      if (N <= 256 && !skinny) return launch_cfg<64, 64, 2, 2, 64, 4, EPI_BF16>(a, s);
      if (skinny) return launch_cfg<64, 128, 2, 2, 64, 4, EPI_BF16>(a, s);
      return launch_cfg<128, 128, 2, 2, 64, 2, EPI_BF16>(a, s);
    case EPI_F32:
      // the LM head: with few rows it streams the weights, so 64x64 tiles
      // (two workgroups per CU, twice the loads in flight); with many rows
      // it is a plain large GEMM
      if (skinny) return launch_cfg<64, 64, 2, 2, 64, 4, EPI_F32>(a, s);
      if (big) return launch_cfg<256, 256, 2, 4, 64, 2, EPI_F32>(a, s);
      return launch_cfg<128, 128, 2, 2, 64, 2, EPI_F32>(a, s);
    case EPI_RESID:
      // residual projections have few output tiles (N = d).  When the tiles
      // past the last full round would leave most CUs idle, one workgroup
      // per CU runs the whole tiles and shares the rest out stream-K;
      // otherwise one workgroup per tile (measured faster at 512 tiles).
      if (big) {
        const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
        const int rem = tiles % gemm_cu_count();
        return launch_cfg<256, 256, 2, 4, 64, 2, EPI_RESID>(a, s, rem != 0 && rem < gemm_cu_count() / 2 ? gemm_cu_count() : 0);
      }
      if (skinny) return launch_cfg<64, 128, 2, 2, 64, 4, EPI_RESID>(a, s);
      return launch_cfg<128, 128, 2, 2, 64, 2, EPI_RESID>(a, s);
    case EPI_SWIGLU:
      if (big) {
        // 256-row tiles on the one-wave-per-SIMD kernel where it applies
        auto rows256 = [&](const GemmArgs &x) {
          if (gemm_w4_eligible(lda, ldb, x.M, N, K, EPI_SWIGLU, b_up_row))
            return launch_gemm_w4(x.A, lda, B, ldb, x.C, ldc, x.M, N, K, EPI_SWIGLU, b_up_row, 1.f, stream);
          return launch_cfg<256, 128, 2, 4, 64, 2, EPI_SWIGLU>(x, s);
        };
        // a last tile row of at most 64 rows costs a whole extra round of
        // 256-row tiles when the full tile rows fill whole rounds; those
        // rows then go to a launch of 64-row tiles instead
        const int tn = (N + 127) / 128, full = M / 256, rest = M - full * 256;
        const int cus = gemm_cu_count();
        if (rest > 0 && rest <= 64 && full > 0 &&
            (full * tn + cus - 1) / cus < ((full + 1) * tn + cus - 1) / cus) {
          GemmArgs lo = a;
          lo.M = full * 256;
          if (int r = rows256(lo)) return r;
          GemmArgs hi = a;
          hi.A = A + (size_t)lo.M * lda;
          hi.C = (uint16_t *)C + (size_t)lo.M * ldc;
          hi.M = rest;
          return launch_cfg<64, 64, 2, 2, 64, 4, EPI_SWIGLU>(hi, s);
        }
        return rows256(a);
      }
      if (skinny) return launch_cfg<64, 64, 2, 2, 64, 4, EPI_SWIGLU>(a, s);
      return launch_cfg<128, 64, 2, 2, 64, 2, EPI_SWIGLU>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

// Adapter shrink with K split over `splits` workgroups per 64 x 64 tile:
// fp32 partial sums into P [splits][rows][nr] (the caller reduces them).
int launch_gemm_f32_ksplit(const uint16_t *A, int lda, const uint16_t *B, int ldb, float *P, int M, int N, int K,
                           int splits, void *stream) {
  if (M <= 0 || N <= 0) return 0;
  if (splits < 1 || splits > 65535) return (int)hipErrorInvalidValue;
  GemmArgs a{};
  a.A = A; a.B = B; a.C = P;
  a.lda = lda; a.ldb = ldb; a.ldc = N; a.M = M; a.N = N; a.K = K;
  a.alpha = 1.f;
  return launch_cfg<64, 64, 2, 2, 64, 4, EPI_F32>(a, (hipStream_t)stream, 0, splits);
}

// The fused QKV epilogue needs head dim 128 and q and k/v sections of whole
// 256-column tiles; below 512 rows the projection takes smaller tiles.
bool qkv_rope_fusable(int M, int Hq, int Hkv, int hd) {
  return hd == 128 && M >= 512 && Hq % 2 == 0 && Hkv % 2 == 0 && Hkv > 0;
}

int launch_gemm_qkv_rope(const uint16_t *A, int lda, const uint16_t *B, int ldb, uint16_t *qkv, int ldc, int M,
                         int K, const LoraArgs *lora, const RopeKv &rk, void *stream) {
  if (!qkv_rope_fusable(M, rk.n_q_heads, rk.n_kv_heads, 128) || !rk.cs || !rk.slot || !rk.kc || !rk.vc ||
      rk.page_size <= 0 || ldc != (rk.n_q_heads + 2 * rk.n_kv_heads) * 128)
    return (int)hipErrorInvalidValue;
  GemmArgs a{};
  a.A = A; a.B = B; a.C = qkv;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc; a.M = M; a.N = ldc; a.K = K;
  a.alpha = 1.f;
  if (lora && lora->U && lora->rows > 0 && lora->r > 0) {
    a.U = lora->U; a.Bx = lora->Bx; a.ldu = lora->ldu; a.r = lora->r; a.lrows = lora->rows;
    a.sec1 = lora->sec1; a.sec2 = lora->sec2;
  }
  a.rope_cs = rk.cs; a.slot = rk.slot; a.kc = rk.kc; a.vc = rk.vc;
  a.q_cols = rk.n_q_heads * 128; a.kv_cols = rk.n_kv_heads * 128; a.n_kv = rk.n_kv_heads; a.ps = rk.page_size;
  return launch_cfg<256, 256, 2, 4, 64, 2, EPI_QKV>(a, (hipStream_t)stream);
}

}  // namespace orthrus
