// Ragged causal attention over the paged KV cache: one launch over a work
// list that mixes chunk tiles (embedding and prefill chunks) and decode
// splits (single-row items), then the log-sum-exp combine of the decode
// rows whose keys were split.
//
// Efficient Iterative Retrieval with Heterogeneous Batching: §3.2 Batch
// Unit (embedding chunks, prefill chunks and decode rows share one pass and
// differ only in length), §2.2 Generation (a decode step reads the cached
// KV of all earlier tokens — memory-bound — while chunk rows are a dense,
// compute-bound pass), §1 and §2.3 (chunks of one request are processed
// across iterations; a later chunk attends to the KV its earlier chunks
// left in the cache).  Row j of an item with context c sits at position
// c + j and sees keys 0 .. c + j; query head h reads KV head h / (Hq/Hkv).
//
// Work entries (built on the host):
//  CHUNK  : 128 (token, head) rows of one item and KV head.  Scores are
//           formed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMAs with K
//           staged in LDS; P^T stays in registers and O^T = V^T P^T reads a
//           transposed V tile from LDS.  Online softmax in fp32 (exp2).
//  DECODE : one decode row, one KV head, one split of its keys.  Head dims
//           64 and 128: each wave streams 16-key blocks with the loads of
//           its next RING-1 blocks in flight; S^T = K Q^T on 16x16x32 bf16 MFMAs
//           (the grouped query heads are the 16 columns), P passes through
//           LDS to the V layout and P.V runs as packed bf16 dot products
//           over key pairs.  Head dims 16 and 32: each wave loads its 32
//           keys at once (HD/8 lanes per key) and scores with packed dot
//           products.  The four waves merge in LDS and write one (max, sum,
//           unnormalised output) partial, or the finished output when one
//           split covers the whole context.
#include "device_common.h"
#include "orthrus_internal.h"

#include <type_traits>

namespace orthrus {

struct AttnArgs {
  const uint16_t *qkv;
  const uint16_t *kc;
  const uint16_t *vc;
  const int32_t *page_ids;
  const AttnWork *work;
  float *part_ml;
  float *part_o;
  uint16_t *o;
  int ld_qkv, ld_o, Hq, Hkv, ps;
  int ps_log2;  // log2(ps) when ps is a power of two, else -1
  float scale_log2;
};

// page index and in-page offset of a key (shifts for power-of-two pages;
// the branch is uniform over the launch)
__device__ __forceinline__ int page_of(const AttnArgs &a, int key) {
  return a.ps_log2 >= 0 ? key >> a.ps_log2 : key / a.ps;
}
__device__ __forceinline__ int slot_of(const AttnArgs &a, int key) {
  return a.ps_log2 >= 0 ? key & (a.ps - 1) : key % a.ps;
}

constexpr int CKT = 64;  // keys per chunk-path tile
constexpr float CHUNK_RESCALE_LOG2 = 8.f;  // lazy-rescale threshold of the chunk path (log2 units)

// Chunk-path LDS: two buffers of one 64-key tile of K and of V, both in
// the cache's [key][head dim] order with 16-byte chunks swizzled per key.
// V rows are padded with zeros to 32 dims for head dims below 32.
template <int HD>
struct ChunkSmem {
  static constexpr int VD = HD < 32 ? 32 : HD;
  uint16_t K[2][CKT * HD];
  uint16_t V[2][CKT * VD];
};
// every buffer starts on a 256-byte boundary of a 256-byte aligned struct
static_assert((CKT * 16 * 2) % 256 == 0, "K and V buffers of every head dim are 256-byte multiples");

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// 32-bit LDS address of a shared-memory object
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS stores of this thread have landed, then the workgroup barrier; no
// wait on global loads in flight (which __syncthreads' fence would add),
// and a compiler barrier for LDS accesses
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte chunk swizzle of a V row.  One 32-lane cycle of
// ds_read_b64_tr_b16 reads 4 consecutive keys x 2 groups of 16 dims (4
// chunks per key); XOR with 4 (key & 3) (rows of 16 chunks, all starting on
// bank 0) or 4 ((key >> 1) & 1) (rows of 8 chunks, odd rows on bank 32)
// gives those 16 chunks 16 distinct 4-bank groups.  Rows of 4 chunks
// already start on 4 different bank quarters.
template <int VCH>
__device__ __forceinline__ int vswz(int key) {
  return VCH >= 16 ? 4 * (key & 3) : VCH == 8 ? 4 * ((key >> 1) & 1) : 0;
}

// Chunk work: 128 (token, head) rows of one item and KV head (32 query
// rows per wave), keys in 64-key tiles.  The K and V chunks of tile t+1 are
// loaded into registers (and the page ids of tile t+2 looked up) while tile
// t is consumed from LDS; one barrier per tile publishes the next buffer.
//  S^T = K Q^T    : 32x32x16 MFMAs, K rows from LDS (ds_read_b128), Q^T in
//                   registers for the whole item.
//  softmax        : online, fp32, exp2 domain, per query row (lane column),
//                   rescaled lazily (only when a row's max grows by more
//                   than 8 in log2 units).
//  O^T += V^T P^T : P^T is the S^T accumulator packed to bf16 (its key
//                   order within a 16-key step is 4h..4h+3, 8+4h..8+4h+3 for
//                   lane half h); the V^T operand takes exactly those keys
//                   with two ds_read_b64_tr_b16, whose 16-lane groups turn
//                   4 keys x 4 dims per lane into 4 keys of one dim per lane
//                   (V rows swizzled so that those reads meet no bank twice).
template <int HD>
__device__ void chunk_path(const AttnArgs &a, const AttnWork &w, ChunkSmem<HD> &sm) {
  constexpr int NCH = HD / 8;                       // 16-byte chunks per K row
  constexpr int VD = ChunkSmem<HD>::VD;
  constexpr int VCH = VD / 8;                       // chunks per V row
  constexpr int NDB = VD / 32;                      // 32-dim blocks of O^T
  constexpr int NLD = (CKT * NCH + 255) / 256;      // chunks per thread per tile (each of K and V)
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;
  const int r = wave * 32 + (lane & 31);
  const int tok = w.q0 + r / G;
  const int head = w.kvh * G + r % G;
  const bool rvalid = (r / G) < w.qn;
  const int rpos = w.ctx + tok;
  const int nkeys = w.ctx + w.q0 + w.qn;
  const int ntiles = (nkeys + CKT - 1) / CKT;
  const int32_t *pages = a.page_ids + w.page_off;

  bf16x8_t q[HD / 16];
  {
    const uint16_t *qrow = a.qkv + (size_t)(w.row0 + (rvalid ? tok : 0)) * a.ld_qkv + head * HD;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (rvalid) v = *(const u32x4_t *)(qrow + kk * 16 + half * 8);
      q[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  if (HD < 32) {  // V dims HD..31 stay zero in both buffers
    for (int c = tid; c < 2 * CKT * (VD - HD) / 8; c += 256) {
      const int b = c / (CKT * (VD - HD) / 8), rem = c % (CKT * (VD - HD) / 8);
      const int key = rem / ((VD - HD) / 8), ch = NCH + rem % ((VD - HD) / 8);
      *(u32x4_t *)(&sm.V[b][key * VD + ch * 8]) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // this thread's chunks of a tile: chunk i = tid + 256 j is key
  // kj0 + KJS j (kj0 = tid / NCH, KJS = 256 / NCH), head-dim chunk
  // cj = tid % NCH; keys past the item re-read its last key.  KJS is a
  // multiple of NCH and of 4 (HD <= 128), so the K swizzle (key mod NCH) and
  // the V swizzle (key mod 4) are the same for every j: a chunk's LDS slot
  // is one per-thread base plus j KJS rows.
  constexpr int KJS = 256 / NCH;
  static_assert(KJS % NCH == 0 && KJS % 4 == 0, "swizzle is per thread");
  const int kj0 = tid / NCH, cj = tid % NCH;
  u32x4_t kreg[NLD], vreg[NLD];
  int pg[NLD];
  auto chunk_ok = [&](int j) { return NLD * 256 == CKT * NCH || tid + 256 * j < CKT * NCH; };
  // Power-of-two pages of at most 64 keys split every whole tile evenly:
  // chunk j of tile t then sits in page t * ppt + (its key in the tile) /
  // ps at a fixed slot, so its offset is page id x page stride plus a
  // per-thread constant.  Other page sizes, and the last tile (clamped
  // keys), take the general per-key form.
  const bool fast = a.ps_log2 >= 0 && a.ps <= CKT;
  const int ppt = fast ? CKT >> a.ps_log2 : 0;
  const uint32_t pstride = (uint32_t)a.Hkv * a.ps * HD;  // elements per page of one layer
  auto whole = [&](int t) { return fast && (t + 1) * CKT <= nkeys; };
  auto lookup = [&](int t) {
    if (whole(t)) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (chunk_ok(j)) pg[j] = pages[t * ppt + ((kj0 + KJS * j) >> a.ps_log2)];
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (chunk_ok(j)) pg[j] = pages[page_of(a, min(t * CKT + kj0 + KJS * j, nkeys - 1))];
    }
  };
  auto load = [&](int t) {
    if (whole(t)) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if (!chunk_ok(j)) continue;
        const int slot = (kj0 + KJS * j) & (a.ps - 1);
        const size_t off = (size_t)(uint32_t)pg[j] * pstride + (uint32_t)((w.kvh * a.ps + slot) * HD + cj * 8);
        kreg[j] = *(const u32x4_t *)(a.kc + off);
        vreg[j] = *(const u32x4_t *)(a.vc + off);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if (!chunk_ok(j)) continue;
        const int p = min(t * CKT + kj0 + KJS * j, nkeys - 1);
        const size_t off = (((size_t)pg[j] * a.Hkv + w.kvh) * a.ps + slot_of(a, p)) * HD + cj * 8;
        kreg[j] = *(const u32x4_t *)(a.kc + off);
        vreg[j] = *(const u32x4_t *)(a.vc + off);
      }
    }
  };
  // LDS byte addresses: the buffers start on 256-byte boundaries, so the
  // XOR terms below (bits 4..7 of a row) never meet the row, block or
  // buffer bits and can be applied after adding those
  const uint32_t k_lds = lds_addr(&sm.K[0][0]), v_lds = lds_addr(&sm.V[0][0]);
  const uint32_t st_k = 2u * (kj0 * HD + ((cj ^ (kj0 & (NCH - 1))) * 8));
  const uint32_t st_v = 2u * (kj0 * VD + ((cj ^ vswz<VCH>(kj0)) * 8));
  auto store = [&](int b) {
    const uint32_t kb_ = k_lds + b * (CKT * HD * 2) + st_k, vb_ = v_lds + b * (CKT * VD * 2) + st_v;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      if (!chunk_ok(j)) continue;
      *(lds_u32x4_t *)(kb_ + j * (KJS * HD * 2)) = kreg[j];
      *(lds_u32x4_t *)(vb_ + j * (KJS * VD * 2)) = vreg[j];
    }
  };
  // K operand of key row (lane & 31) of a 32-key block, head-dim chunk
  // 2 kk + half, swizzled by x = lane mod NCH: with x' = x / 2 its element
  // index is (row HD + 16 x' + 8 (half ^ (x & 1))) XOR 16 kk
  const int xk = lane & (NCH - 1);
  const uint32_t k_rd = 2u * ((lane & 31) * HD + 16 * (xk >> 1) + 8 * (half ^ (xk & 1)));
  // V^T operand (ds_read_b64_tr_b16): key 4 half + jj / 4 of an 8-key
  // group, dims 32 db + 16 (g & 1) + 4 (jj & 3) ..; the row swizzle c (a
  // multiple of 4 chunks) turns the index into
  // (key VD + 32 (c / 4) + 8 u + 4 (jj & 1)) XOR 32 db, u = 2 (g & 1) + (jj & 3) / 2
  const int g = lane >> 4, jj = lane & 15;
  const int vkey = 4 * half + (jj >> 2);
  const int vu = 2 * (g & 1) + ((jj & 3) >> 1);
  const uint32_t v_rd = 2u * (vkey * VD + 32 * (vswz<VCH>(vkey) >> 2) + 8 * vu + 4 * (jj & 1));

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int min_rpos = w.ctx + w.q0;

  lookup(0);
  load(0);
  if (ntiles > 1) lookup(1);
  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    store(b);
    if (t + 1 < ntiles) {
      load(t + 1);
      if (t + 2 < ntiles) lookup(t + 2);
    }
    lds_barrier();
    const int kt0 = t * CKT;
    const uint32_t kt = k_lds + b * (CKT * HD * 2) + k_rd;
    const uint32_t vt = v_lds + b * (CKT * VD * 2) + v_rd;

    // S^T for the tile's two 32-key blocks
    f32x16_t s[CKT / 32];
#pragma unroll
    for (int kb = 0; kb < CKT / 32; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk) {
        const bf16x8_t kop =
            __builtin_bit_cast(bf16x8_t, *(const lds_u32x4_t *)((kt ^ (32u * kk)) + kb * (32 * HD * 2)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, q[kk], s[kb], 0, 0, 0);
      }
    }
    // causal mask (only tiles that reach past the first row's position
    // need it; it also hides the clamped keys past the item) and the tile
    // max of the raw scores; the scale (> 0) is applied to the max and
    // folded into the exponent below.  Query rows past the chunk compute on
    // zero q and are never written.
    float mt = -INFINITY;
    if (kt0 + CKT - 1 > min_rpos) {
#pragma unroll
      for (int kb = 0; kb < CKT / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt0 + kb * 32 + (e / 4) * 8 + half * 4 + (e % 4);
          const float v = key > rpos ? -INFINITY : s[kb][e];
          s[kb][e] = v;
          mt = fmaxf(mt, v);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < CKT / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, s[kb][e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * a.scale_log2;
    // lazy rescaling: the running max (and with it l and the output
    // accumulators) moves only when some row of the wave meets a tile max
    // above it by more than CHUNK_RESCALE_LOG2; otherwise the stale max
    // stays and p = 2^(s c - m) stays below 2^CHUNK_RESCALE_LOG2, which bf16
    // P and the fp32 sums hold without loss.  The first tile always moves
    // it (every row sees key 0).
    if (__builtin_amdgcn_ballot_w64(mt > m_run + CHUNK_RESCALE_LOG2) != 0) {  // uniform over the wave
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < CKT / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[kb][e], a.scale_log2, -m_use));
        s[kb][e] = pr;
        lsum += pr;
      }
    l_run += lsum;

    // O^T += V^T P^T in 16-key steps
#pragma unroll
    for (int st = 0; st < CKT / 16; ++st) {
      const int kb = st / 2, e0 = (st % 2) * 8;
      bf16x8_t pop;  // v_cvt_pk_bf16_f32, round to nearest even
#pragma unroll
      for (int i = 0; i < 8; ++i) pop[i] = (__bf16)s[kb][e0 + i];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x2_t vv[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const uint32_t src = (vt ^ (64u * db)) + (st * 16 + rr * 8) * (VD * 2);
          const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)src);
          vv[rr] = __builtin_bit_cast(u32x2_t, v);
        }
        u32x4_t vw;
        vw[0] = vv[0][0]; vw[1] = vv[0][1]; vw[2] = vv[1][0]; vw[3] = vv[1][1];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pop, oacc[db], 0, 0, 0);
      }
    }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!rvalid) return;
  const float inv = 1.f / l_tot;
  uint16_t *orow = a.o + (size_t)(w.row0 + tok) * a.ld_o + head * HD;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + half * 4;
      if (d >= HD) continue;
      uint2 wv;
      wv.x = pack_bf2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv);
      wv.y = pack_bf2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv);
      *(uint2 *)(orow + d) = wv;
    }
}

// DPP helpers: sums over the 2/4/8/16 lanes of one key within a 16-lane
// row without going through the LDS crossbar.  quad_perm [1,0,3,2] and
// [2,3,0,1] exchange lanes 1 and 2 apart; row_half_mirror pairs lane i with
// 7-i (the other quad of the half-row); row_mirror pairs i with 15-i (the
// other half of the row).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int LPK>
__device__ __forceinline__ float key_sum(float v) {
  if (LPK >= 2) v += dpp<0xB1>(v);
  if (LPK >= 4) v += dpp<0x4E>(v);
  if (LPK >= 8) v += dpp<0x141>(v);
  if (LPK >= 16) v += dpp<0x140>(v);
  return v;
}

template <int HD, int G>
struct DecodeSmem {
  float o[ATTN_WAVES][G * HD];
  float ml[ATTN_WAVES][G][2];
  int pages[DEC_SPLIT_VEC + 2];
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// q_pair . k_pair in fp32 (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t q2, uint32_t k2, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q2), __builtin_bit_cast(bf16x2_t, k2), c,
                                         false);
}

// Merge the four waves' (max, sum, unnormalised output) records of one
// decode split and write either the finished output row (the split covers
// the whole context) or the split's partial for the combine kernel.
template <int HD, int G>
__device__ void finish_decode(const AttnArgs &a, const AttnWork &w,
                              const float (*o)[G * HD], const float (*ml)[G][2]) {
  const bool whole = (w.k0 == 0 && w.k1 == w.ctx + 1);
  for (int t = threadIdx.x; t < G * HD; t += 256) {
    const int h = t / HD, d = t % HD;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < ATTN_WAVES; ++v) M = fmaxf(M, ml[v][h][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < ATTN_WAVES; ++v) {
      if (ml[v][h][0] == -INFINITY) continue;  // a wave with no keys
      const float wgt = exp2f(ml[v][h][0] - M);
      L += wgt * ml[v][h][1];
      O += wgt * o[v][t];
    }
    if (whole) {
      a.o[(size_t)w.row0 * a.ld_o + (w.kvh * G + h) * HD + d] = (uint16_t)f2bf(O / L);
    } else {
      a.part_o[((size_t)w.part * G + h) * HD + d] = O;
      if (d == 0) {
        a.part_ml[((size_t)w.part * G + h) * 2 + 0] = M;
        a.part_ml[((size_t)w.part * G + h) * 2 + 1] = L;
      }
    }
  }
}

// Decode work: keys [k0, k1) (at most 128) of one decode row and one KV
// head.  The split's page ids are staged in LDS once.  Each wave takes 32
// keys and issues all of their K and V loads before any arithmetic (HD/8
// lanes per key, 16-byte loads over the contiguous page_size x HD blocks),
// scores all grouped query heads with packed bf16 dot products, and the
// four waves merge in LDS: one partial per workgroup, or the final output
// when this split covers the whole context.
template <int HD, int G>
__device__ void decode_path(const AttnArgs &a, const AttnWork &w, DecodeSmem<HD, G> &sm) {
  constexpr int LPK = HD / 8;                  // lanes per key
  constexpr int KPI = 64 / LPK;                // keys per wave load
  constexpr int WK = DEC_SPLIT_VEC / ATTN_WAVES;  // keys per wave
  constexpr int NL = WK / KPI > 0 ? WK / KPI : 1;
  static_assert(NL * KPI >= WK, "wave key span");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kg = lane / LPK;
  const int pi0 = page_of(a, w.k0);
  const int npg = page_of(a, w.k1 - 1) - pi0 + 1;
  for (int t = threadIdx.x; t < npg; t += 256) sm.pages[t] = a.page_ids[w.page_off + pi0 + t];
  __syncthreads();
  const int wk0 = w.k0 + wave * WK;
  const int wk1 = min(w.k1, wk0 + WK);
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  if (wk0 < wk1) {
    // all loads first; lanes past the end re-read the last key (masked)
    u32x4_t kr[NL], vr[NL];
    const size_t head_off = (size_t)w.kvh * a.ps;
#pragma unroll
    for (int li = 0; li < NL; ++li) {
      const int key = min(wk0 + li * KPI + kg, wk1 - 1);
      const int page = sm.pages[page_of(a, key) - pi0];
      const size_t off = (((size_t)page * a.Hkv * a.ps) + head_off + slot_of(a, key)) * HD + sub * 8;
      kr[li] = *(const u32x4_t *)(a.kc + off);
      vr[li] = *(const u32x4_t *)(a.vc + off);
    }
    u32x4_t q[G];
    const uint16_t *qrow = a.qkv + (size_t)w.row0 * a.ld_qkv + (w.kvh * G) * HD + sub * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) q[h] = *(const u32x4_t *)(qrow + h * HD);
    float sc[NL][G];
#pragma unroll
    for (int li = 0; li < NL; ++li) {
      const bool valid = wk0 + li * KPI + kg < wk1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = dot2(q[h][0], kr[li][0], 0.f);
        d = dot2(q[h][1], kr[li][1], d);
        d = dot2(q[h][2], kr[li][2], d);
        d = dot2(q[h][3], kr[li][3], d);
        d = key_sum<LPK>(d) * a.scale_log2;
        sc[li][h] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int li = 1; li < NL; ++li) mx = fmaxf(mx, sc[li][h]);
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      m[h] = mx;  // finite: the wave has at least one valid key
#pragma unroll
      for (int li = 0; li < NL; ++li) {
        const float pr = exp2f(sc[li][h] - mx);
        l[h] += pr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h][2 * e] = fmaf(pr, lo_bf(vr[li][e]), acc[h][2 * e]);
          acc[h][2 * e + 1] = fmaf(pr, hi_bf(vr[li][e]), acc[h][2 * e + 1]);
        }
      }
    }
  }
  // sum the key groups (each LPK-lane group saw different keys) and stage
  // this wave's (m, l, o) in LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float lt = l[h];
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) lt += __shfl_xor(lt, o, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[h][e] = v;
    }
    if (kg == 0) {
      float *dst = &sm.o[wave][h * HD + sub * 8];
      *(float4 *)dst = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *(float4 *)(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (lane == 0) {
      sm.ml[wave][h][0] = m[h];
      sm.ml[wave][h][1] = lt;
    }
  }
  __syncthreads();
  finish_decode<HD, G>(a, w, sm.o, sm.ml);
}

// Decode work, head dims 64 and 128: keys [k0, k1) (at most DEC_SPLIT_MAX)
// of one decode row and one KV head.  The split's page ids are staged in
// LDS once.  Wave w walks the 16-key blocks w, w + 4, ... with the K and V
// loads of its next block in flight while the current block is consumed.
//  - K operand: lane l holds key l % 16 of the block, head-dim chunk
//    (l / 16) + 4 j for k-slice j; Q^T is the B operand with the G grouped
//    heads as columns (slots G..15 zero).  The 16x16 fp32 result gives lane
//    l the scores of keys 4 (l / 16) .. +3 for head l % 16.
//  - Online softmax per head in the score layout: the block maximum over
//    the four lane groups, the rescale factor alpha and p = 2^(s - m).
//  - p and alpha go through a per-wave LDS slot to the V layout (lane l:
//    head-dim chunk l % (HD/8), keys NL (l / (HD/8)) .. +NL-1), where the
//    accumulators are rescaled only when some alpha differs from 1 and
//    P.V runs as v_dot2 over (p_i, p_i+1) x (v_i, v_i+1) pairs, p rounded
//    to bf16 like the P operand of the chunk path.
template <int HD, int G>
struct DecodeMfmaSmem {
  float o[ATTN_WAVES][G * HD];
  float ml[ATTN_WAVES][G][2];
  float pb[ATTN_WAVES][G][16];
  float al[ATTN_WAVES][16];
  int pages[DEC_SPLIT_MAX + 2];
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int HD, int G, int RING>
__device__ void decode_mfma_path(const AttnArgs &a, const AttnWork &w, DecodeMfmaSmem<HD, G> &sm) {
  static_assert(HD == 64 || HD == 128, "head dim");
  constexpr int LPK = HD / 8;   // lanes per key row in the V layout
  constexpr int KPI = 64 / LPK; // key groups of the V layout
  constexpr int NL = 16 / KPI;  // keys per lane per block (V)
  constexpr int NJ = HD / 32;   // MFMA k-slices
  static_assert(NL % 2 == 0, "key pairs");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pi0 = page_of(a, w.k0);
  const int npg = page_of(a, w.k1 - 1) - pi0 + 1;
  for (int t = threadIdx.x; t < npg; t += 256) sm.pages[t] = a.page_ids[w.page_off + pi0 + t];
  const int qh = lane & 15, qg = lane >> 4;
  u32x4_t q[NJ];
  {
    const uint16_t *qrow =
        a.qkv + (size_t)w.row0 * a.ld_qkv + (size_t)(w.kvh * G + (qh < G ? qh : 0)) * HD + qg * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (qh < G) v = *(const u32x4_t *)(qrow + j * 32);
      q[j] = v;
    }
  }
  __syncthreads();
  const int sub = lane % LPK, kg = lane / LPK;
  const int nblk = (w.k1 - w.k0 + 15) / 16;
  float m_run = -INFINITY, l_part = 0.f;
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  auto row_off = [&](int key) -> size_t {
    const int page = sm.pages[page_of(a, key) - pi0];
    return (((size_t)page * a.Hkv + w.kvh) * a.ps + slot_of(a, key)) * HD;
  };
  // keys past the split re-read its last key; their scores are masked
  auto issue = [&](int b, u32x4_t *kr, u32x4_t *vr) {
    const int base = w.k0 + b * 16;
    const size_t ko = row_off(min(base + qh, w.k1 - 1)) + qg * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) kr[j] = *(const u32x4_t *)(a.kc + ko + j * 32);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      vr[i] = *(const u32x4_t *)(a.vc + row_off(min(base + kg * NL + i, w.k1 - 1)) + sub * 8);
  };
  auto consume = [&](int b, const u32x4_t *kr, const u32x4_t *vr) {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[j]),
                                                     __builtin_bit_cast(bf16x8_t, q[j]), sacc, 0, 0, 0);
    const int key0 = w.k0 + b * 16 + 4 * qg;
    float sc[4], mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = key0 + e < w.k1 ? sacc[e] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sc[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: every block has a valid key
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float p[4], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = exp2f(sc[e] - m_new);
      psum += p[e];
    }
    l_part = l_part * alpha + psum;
    if (qh < G) {
      *(float4 *)&sm.pb[wave][qh][4 * qg] = make_float4(p[0], p[1], p[2], p[3]);
      if (qg == 0) sm.al[wave][qh] = alpha;
    }
    wave_lds_sync();
    float alh[G];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      alh[h] = sm.al[wave][h];
      rescale |= alh[h] != 1.f;
    }
    if (rescale) {  // uniform: every lane read the same factors
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alh[h];
    }
    // (v_i[d], v_i+1[d]) pairs: low halves, then high halves of each word
    uint32_t x[NL / 2][8];
#pragma unroll
    for (int pr = 0; pr < NL / 2; ++pr)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        x[pr][2 * wd] = __builtin_amdgcn_perm(vr[2 * pr + 1][wd], vr[2 * pr][wd], 0x05040100u);
        x[pr][2 * wd + 1] = __builtin_amdgcn_perm(vr[2 * pr + 1][wd], vr[2 * pr][wd], 0x07060302u);
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float pv[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) pv[i] = sm.pb[wave][h][kg * NL + i];
#pragma unroll
      for (int pr = 0; pr < NL / 2; ++pr) {
        const bf16x2_t pk = {(__bf16)pv[2 * pr], (__bf16)pv[2 * pr + 1]};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[h][e] = __builtin_amdgcn_fdot2_f32_bf16(pk, __builtin_bit_cast(bf16x2_t, x[pr][e]), acc[h][e], false);
      }
    }
    wave_lds_sync();  // the slot is rewritten by the next block
  };
  // a ring of RING blocks in registers: RING-1 blocks in flight while one
  // is consumed (the wave takes blocks wave, wave + 4, ...)
  u32x4_t kb[RING][NJ], vb[RING][NL];
  int b = wave;
#pragma unroll
  for (int r = 0; r < RING - 1; ++r)
    if (b + r * ATTN_WAVES < nblk) issue(b + r * ATTN_WAVES, kb[r], vb[r]);
  while (b < nblk) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      if (b < nblk) {
        const int nb = b + (RING - 1) * ATTN_WAVES;
        if (nb < nblk) issue(nb, kb[(r + RING - 1) % RING], vb[(r + RING - 1) % RING]);
        consume(b, kb[r], vb[r]);
      }
      b += ATTN_WAVES;
    }
  }
  // totals over the lane groups, then stage this wave's record
  float lt = l_part + __shfl_xor(l_part, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int o = LPK; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[h][e] = v;
    }
    if (kg == 0) {
      float *dst = &sm.o[wave][h * HD + sub * 8];
      *(float4 *)dst = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *(float4 *)(dst + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (qh < G && qg == 0) {
    sm.ml[wave][qh][0] = m_run;  // -inf for a wave with no block
    sm.ml[wave][qh][1] = lt;
  }
  __syncthreads();
  finish_decode<HD, G>(a, w, sm.o, sm.ml);
}

// One launch over the whole work list: each workgroup runs the chunk path
// or the decode path of its entry, so the HBM-bound decode splits and the
// matrix-bound chunk tiles of one step share the chip.  The launch takes the
// chunk path's registers and LDS (two workgroups per CU at head dim 128);
// the decode path uses the spare registers for a 4-block load ring (2 where
// 8 grouped heads at head dim 128 leave no room).
template <int HD, int G>
union RaggedSmem {
  ChunkSmem<HD> c;
  typename std::conditional<(HD >= 64), DecodeMfmaSmem<HD, G>, DecodeSmem<HD, G>>::type d;
};

template <int HD, int G>
__global__ __launch_bounds__(256, 2) void attn_ragged_kernel(AttnArgs a) {
  // 256-byte alignment: the chunk path's address XORs rely on it
  __shared__ __attribute__((aligned(256))) RaggedSmem<HD, G> sm;
  const AttnWork w = a.work[blockIdx.x];
  if (w.type == WORK_CHUNK) {
    chunk_path<HD>(a, w, sm.c);
  } else {
    if constexpr (HD >= 64) decode_mfma_path<HD, G, (HD == 128 && G == 8) ? 2 : 4>(a, w, sm.d);
    else decode_path<HD, G>(a, w, sm.d);
  }
}

// Merge the split partials of each decode row: out = sum_p 2^(m_p - M) o_p /
// sum_p 2^(m_p - M) l_p.  Grid (decode item, KV head), 256 threads.  The
// per-partial weights of every grouped head are formed once into LDS
// (lanes over partials), then each thread sums its output elements over
// the partials with independent coalesced loads.  Rows whose context fits
// one split were finished by the attention kernel itself.
constexpr int COMB_MAXP = 256;  // partials merged per pass

template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const DevItem *items, const int32_t *dec_items,
                                                           const float *part_ml, const float *part_o,
                                                           uint16_t *o, int ld_o, int G) {
  __shared__ float wts[8][COMB_MAXP];
  __shared__ float Ms[8], Mrun[8], Lrun[8];
  const DevItem it = items[dec_items[blockIdx.x]];
  if (it.n_parts <= 1) return;
  const int kvh = blockIdx.y;
  const int p0 = it.part0 + kvh * it.n_parts;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int PER = (8 * HD + 255) / 256;  // output elements per thread (G <= 8)
  float accs[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) accs[i] = 0.f;
  if (threadIdx.x < 8) {
    Mrun[threadIdx.x] = -INFINITY;
    Lrun[threadIdx.x] = 0.f;
  }
  for (int q0 = 0; q0 < it.n_parts; q0 += COMB_MAXP) {
    const int np = min(COMB_MAXP, it.n_parts - q0);
    __syncthreads();
    // weights of this pass, one wave per head
    for (int h = wave; h < G; h += 4) {
      float M = -INFINITY;
      for (int p = lane; p < np; p += 64) M = fmaxf(M, part_ml[((size_t)(p0 + q0 + p) * G + h) * 2]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
      const float Mnew = fmaxf(M, Mrun[h]);
      float L = 0.f;
      for (int p = lane; p < np; p += 64) {
        const size_t idx = (size_t)(p0 + q0 + p) * G + h;
        const float wgt = exp2f(part_ml[idx * 2] - Mnew);
        wts[h][p] = wgt;
        L += wgt * part_ml[idx * 2 + 1];
      }
      L = wave_sum(L);
      if (lane == 0) {
        Ms[h] = exp2f(Mrun[h] - Mnew);  // rescale of the earlier passes
        Lrun[h] = Lrun[h] * Ms[h] + L;
        Mrun[h] = Mnew;
      }
    }
    __syncthreads();
    // the loads of up to eight partials are issued together, then their
    // fmas run in partial order (np is uniform over the block)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = threadIdx.x + i * 256;
      if (t >= G * HD) break;
      const int h = t / HD;
      float acc = accs[i] * Ms[h];
      const float *src = part_o + (size_t)(p0 + q0) * G * HD + t;
      for (int p = 0; p < np; p += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p + u < np) v[u] = src[(size_t)(p + u) * G * HD];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p + u < np) acc = fmaf(wts[h][p + u], v[u], acc);
      }
      accs[i] = acc;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = threadIdx.x + i * 256;
    if (t >= G * HD) break;
    const int h = t / HD, d = t % HD;
    o[(size_t)it.row0 * ld_o + (kvh * G + h) * HD + d] = (uint16_t)f2bf(accs[i] / Lrun[h]);
  }
}

static AttnArgs attn_args(const uint16_t *qkv, int ld_qkv, const uint16_t *kc, const uint16_t *vc,
                          const int32_t *page_ids, const AttnWork *work, float *part_ml,
                          float *part_o, uint16_t *o, int ld_o, int Hq, int Hkv, int hd, int ps) {
  AttnArgs a;
  a.qkv = qkv; a.kc = kc; a.vc = vc; a.page_ids = page_ids; a.work = work;
  a.part_ml = part_ml; a.part_o = part_o; a.o = o;
  a.ld_qkv = ld_qkv; a.ld_o = ld_o; a.Hq = Hq; a.Hkv = Hkv; a.ps = ps;
  a.ps_log2 = (ps & (ps - 1)) == 0 ? __builtin_ctz((unsigned)ps) : -1;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
  return a;
}

template <int HD>
static int launch_ragged_hd(const AttnArgs &a, int n_work, int G, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_ragged_kernel<HD, 1>), dim3(n_work), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attn_ragged_kernel<HD, 2>), dim3(n_work), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_ragged_kernel<HD, 4>), dim3(n_work), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_ragged_kernel<HD, 8>), dim3(n_work), dim3(256), 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

int launch_attn_ragged(const uint16_t *qkv, int ld_qkv, const uint16_t *kc, const uint16_t *vc,
                       const int32_t *page_ids, const AttnWork *work, int n_work,
                       float *part_ml, float *part_o, uint16_t *o, int ld_o, int Hq, int Hkv, int hd, int ps,
                       void *stream) {
  if (n_work <= 0) return 0;
  const AttnArgs a = attn_args(qkv, ld_qkv, kc, vc, page_ids, work, part_ml, part_o, o, ld_o, Hq, Hkv, hd, ps);
  const int G = Hq / Hkv;
  hipStream_t s = (hipStream_t)stream;
  switch (hd) {
    case 16: return launch_ragged_hd<16>(a, n_work, G, s);
    case 32: return launch_ragged_hd<32>(a, n_work, G, s);
    case 64: return launch_ragged_hd<64>(a, n_work, G, s);
    case 128: return launch_ragged_hd<128>(a, n_work, G, s);
  }
  return (int)hipErrorInvalidValue;
}

int decode_split_limit(int hd) { return hd >= 64 ? DEC_SPLIT_MAX : DEC_SPLIT_VEC; }

int launch_attn_combine(const DevItem *items, const int32_t *dec_items, int n_dec, const float *part_ml,
                        const float *part_o, uint16_t *o, int ld_o, int Hq, int Hkv, int hd,
                        void *stream) {
  if (n_dec <= 0) return 0;
  const int G = Hq / Hkv;
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(n_dec, Hkv);
  switch (hd) {
    case 16: hipLaunchKernelGGL(attn_combine_kernel<16>, grid, dim3(256), 0, s, items, dec_items, part_ml, part_o, o, ld_o, G); break;
    case 32: hipLaunchKernelGGL(attn_combine_kernel<32>, grid, dim3(256), 0, s, items, dec_items, part_ml, part_o, o, ld_o, G); break;
    case 64: hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, s, items, dec_items, part_ml, part_o, o, ld_o, G); break;
    case 128: hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, s, items, dec_items, part_ml, part_o, o, ld_o, G); break;
    default: return (int)hipErrorInvalidValue;
  }
  ORTHRUS_LAUNCH_CHECK();
  return 0;
}

}  // namespace orthrus
