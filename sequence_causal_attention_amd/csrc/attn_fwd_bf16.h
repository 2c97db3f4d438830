// attn_fwd_bf16.h -- causal attention forward of one sequence-parallel rank, bf16 in,
// fp32 accumulation, bf16 MFMA (v_mfma_f32_32x32x16_bf16) for both products.
//
// What is computed ("Folding Tensor and Sequence Parallelism ...", section 2, attention
// layers; "AutoSP ...", section 2.A item 4; "Tensor, pipeline e sequence parallelism",
// section 01, GQA paragraph): for each local query row i of the rank and query head h,
// softmax over the keys j <= g(i) of the scaled scores q_i . k_j / sqrt(dh), applied to
// the values of KV head h / grp; plus lse_i, the natural-log log-sum-exp of the scores.
//
// Design for gfx950 (the pages only name "FlashAttention" on other hardware):
//  * Work unit = one KV head, GH of its query heads, and a mirrored pair of query tiles
//    of BQ local rows (tile n_qtiles-1-p, then tile p). Under the zigzag map a pair needs
//    S_total + BQ keys whatever p and the rank, so all workgroups and all ranks do equal
//    work. Units are laid out so that each XCD gets a contiguous range (same KV head,
//    sweeping the same K/V tiles through that XCD's L2).
//  * A wave owns RB row blocks of 32 query rows. Scores are computed transposed,
//    S^T = K Q^T (keys on MFMA rows, queries on MFMA columns): each lane holds one query
//    column, so row max / row sum are in-lane plus one swap of the two 32-lane halves,
//    and the fp32 accumulator, rounded to bf16, is already the B operand of
//    O^T = V^T P^T. Q^T stays in registers for the whole key sweep.
//  * K/V are staged in 32 * SPS-key stages straight from global memory into LDS
//    (global_load_lds_dwordx4, no register round trip) through a ring of NBUF stages,
//    PD = NBUF-2 stages ahead of use; every wave issues an equal share of each stage and
//    waits (vmcnt) only for the stage it needs next. Rows are XOR-swizzled at 16-byte
//    granularity so both LDS read patterns are bank-conflict free: K as one ds_read_b128
//    per MFMA operand, V^T through the gfx950 transposing read ds_read_b64_tr_b16 (two
//    per MFMA operand), which also makes V's key order match the P operand.
//  * Software pipeline per 32-key step t: the QK^T MFMAs of step t+1 are issued in the
//    same basic block as the exp2/convert/sum VALU work of step t, and the PV MFMAs of
//    step t in the same block as the mask/row-max VALU work of step t+1, so matrix and
//    vector pipes overlap inside one wave.
//  * Causal tile skipping: the sweep stops at the tile's last global position; keys past
//    it are never loaded (loads are clamped to the last needed row). Only steps that
//    reach past a wave's first position apply the element mask (key > position -> -inf).
//  * Online softmax in base 2 (log2(e)/sqrt(dh) folded into one FMA), running max raised
//    lazily (TSP_RESCALE_SLACK), row sums from the rounded bf16 weights (v_dot2).
//  * dh 256 (and dh 128 with two row blocks per wave, which halves the LDS reads per
//    product) runs one wave per SIMD: its Q^T operands and outputs fill the registers, and
//    no second wave covers a wave's own waits. The unrolled steps keep the running max of
//    the sweep's first step (no per-step test and branch; a tile that overflowed is swept
//    again with the test) and are issued in a fixed order: K operands read four operands
//    ahead, the V^T operands and the weights of step t under the QK^T products of step
//    t+1, then the PV products back to back with the stage boundary and the next loads
//    under them.
#pragma once

#include <type_traits>

#include "attn_common.h"

#ifndef TSP_PINGPONG
#define TSP_PINGPONG 1
#endif
#ifndef TSP_RING_SCOPE
#define TSP_RING_SCOPE __HIP_MEMORY_SCOPE_SYSTEM
#endif
#ifndef TSP_PP_LAGGED
#define TSP_PP_LAGGED(w) ((w) >= NW / 2)
#endif

namespace tsp {

typedef __bf16 tsp_bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) tsp_bf16x4* lds_bf16x4_ptr;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations are outstanding and leaves the LDS/export counters alone.
__device__ __forceinline__ void tsp_wait_vmcnt(int n) {
  switch (n) {  // the count must be an immediate
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
    default: __builtin_amdgcn_s_waitcnt(0x4F70); break;  // 16: vmcnt high bits = 1
  }
}

// s_waitcnt with vmcnt = N (0..63), other counters untouched.
template <int N>
__device__ __forceinline__ void tsp_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory straight into LDS: lane i reads sbase + voff
// (sbase wave-uniform, voff its own byte offset) and writes lds_addr + 16*i (gfx950
// global_load_lds_dwordx4, saddr form, LDS base in M0). Issued as inline asm on purpose:
// the compiler then does not track the LDS write and does not wait for every in-flight
// prefetch (vmcnt(0)) before each LDS read; the kernel instead waits for exactly the
// stage it is about to read (vmcnt + barrier).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void tsp_lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t tsp_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

template <int DH, int NW, int NBUF, int SPS>
struct Bf16Stage {
  static constexpr int BK = 32;                       // keys per pipeline step
  static constexpr int BKS = BK * SPS;                // keys per stage (one wait + barrier)
  static constexpr int ROW_BYTES = DH * 2;            // one K or V row
  static constexpr int CPR = DH / 8;                  // 16-byte chunks per row
  static constexpr int RPL = 64 / CPR;                // rows per 1 KiB wave-load
  static constexpr int TILE_BYTES = BKS * ROW_BYTES;  // one K (or V) tile of a stage
  static constexpr int WL = TILE_BYTES / 1024;       // wave-loads per K (or V) tile
  static constexpr int LPW = 2 * WL / NW;            // wave-loads per wave per stage
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  // Ring layout: the K tiles of all slots first, then the V tiles, so four of the five
  // slots of each lie within the 16-bit DS offset of one per-lane base register (no
  // address add per read).
  static constexpr int SLOT_STRIDE = TILE_BYTES;
  static constexpr int V_BASE = NBUF * TILE_BYTES;
  static constexpr int PD = NBUF - 2;                // prefetch distance in stages
  static constexpr int SWZ = CPR < 16 ? CPR : 16;    // swizzle period (chunks)
  static_assert((2 * WL) % NW == 0, "stage loads must split evenly over the waves");
  static_assert(LPW * PD <= 16, "vmcnt range");
  static_assert(CPR >= 8, "head dim");
  // XOR swizzles on the 16-byte chunk index of a row (row = key index in the stage).
  // K: lanes reading 16 consecutive rows at one logical chunk hit 16 distinct chunks.
  __device__ static int swz_k(int row) { return row & (SWZ - 1); }
  // V: a 16-lane group of the transposing read takes one chunk pair (32 bytes) from each
  // of 4 consecutive rows, and the next group the adjacent pair of the same rows. XOR-ing
  // the chunk index with 4*(row%4) keeps pairs whole and spreads those 8 (row, pair)
  // reads over 8 distinct 32-byte bank groups. With 128-byte rows (dh 64) two rows share
  // one 256-byte bank line, so the row's second bit picks the XOR instead.
  __device__ static int swz_v(int row) { return CPR >= 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};

// NR: key ranges of the launch, 1 ([kv_lo, kv_hi)) or 2 (also [kv_lo2, kv_hi2), after the
// first): one sweep runs through both, the second range's stages following the first's in
// the LDS ring, so the pipeline neither drains nor refills between them.
// NR = 3 is the ring sweep over the peers' chunks: for ring steps s = 1 .. D-1 the chunks
// p and 2D-1-p of peer p = (rank - s) mod D, in that order, each taken whole by a tile
// whose rows lie in a later chunk and skipped otherwise (no chunk straddles a row's
// position, so nothing is masked). The sweep runs over a virtual key axis (the visible
// chunks back to back); each stage's physical keys come from the chunk cursor, which also
// waits for the chunk's arrival flag before the first stage of a chunk is loaded.
#ifndef TSP_FWD_FIXED_MAX
#define TSP_FWD_FIXED_MAX 1
#endif
#ifndef TSP_FWD_PINNED
#define TSP_FWD_PINNED 1
#endif
#ifndef TSP_PIN_KW
#define TSP_PIN_KW 0  // 0: 4 K operands ahead with one row block, 2 with two
#endif
#ifndef TSP_PIN_BJ
#define TSP_PIN_BJ 3
#endif
#ifndef TSP_PIN_SPLIT
#define TSP_PIN_SPLIT 1
#endif
template <int DH, int NW, int RB, int NBUF, int SPS, int OCC, int NR>
__global__ __launch_bounds__(NW * 64, OCC) void attn_fwd_bf16_kernel(TspParams p) {
  using St = Bf16Stage<DH, NW, NBUF, SPS>;
  constexpr int BK = St::BK;
  constexpr int NDB = DH / 32;  // 32-dim blocks of the output
  constexpr int NKK = DH / 16;  // reduction steps of QK^T
  constexpr int PD = St::PD;
  // One wave per SIMD with 256 output dims per row block pair or more (dh 256, or dh 128 with
  // two row blocks), where the per-step test costs most: the unrolled steps keep the
  // running max of the sweep's first step instead of testing every step's scores against it.
  // Their weights are then 2^(x - m) with m at most the row's true max, exact up to overflow;
  // a tile whose sums or outputs left the finite range is swept again with the test on
  // every step.
  constexpr bool FIXED_MAX = OCC == 1 && RB * DH >= 256 && NR != 3 && TSP_FWD_FIXED_MAX;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * St::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);
  uint16_t* __restrict__ og = static_cast<uint16_t*>(p.out);

  // ---- which unit of work ------------------------------------------------------------
  int32_t unit = tsp_xcd_unit(blockIdx.x, gridDim.x);
  const int32_t pair = unit % p.n_pairs;
  unit /= p.n_pairs;
  const int32_t hgrp = unit % p.n_hgroups;
  unit /= p.n_hgroups;
  const int32_t hk = unit % p.Hkv;
  const int32_t b = unit / p.Hkv;

  const int64_t kv_row_stride = p.kv_stride;  // elements between consecutive keys
  const int pos_blocks = p.BQ / 32;  // row blocks per head in a tile

  // ---- per-lane LDS read offsets (constant over the sweep) ------------------------------
  // K operand of QK^T step kk: row `col`, logical chunk 2kk + half. With FIXED_MAX (its
  // registers are short), one offset per swizzle period: chunks SWZ apart lie SWZ * 16
  // bytes apart, so KP (VP) offsets serve all NKK (NDB) operands.
  constexpr int KP = FIXED_MAX && NKK > St::SWZ / 2 ? St::SWZ / 2 : NKK;
  constexpr int VP = FIXED_MAX && NDB > St::SWZ / 4 ? St::SWZ / 4 : NDB;
  int koff[KP];
#pragma unroll
  for (int kk = 0; kk < KP; ++kk) koff[kk] = col * St::ROW_BYTES + (((2 * kk + half) ^ St::swz_k(col)) << 4);
  // V^T operand of PV block db: in each 16-lane group g, source lane s addresses row
  // 4*half + s/4 (+16 per 16-key step, +8 for the second read) and dims
  // db*32 + 16(g&1) + 4(s&3) .. +3; lane s then receives dim db*32 + 16(g&1) + s of the
  // 4 rows, which is the A operand layout with keys in the P operand's order.
  int voff[VP];
  {
    const int g = lane >> 4, s = lane & 15;
    const int vrow = 4 * half + (s >> 2);
    const int xv = St::swz_v(vrow);  // rows +8 and +16 have the same swizzle
#pragma unroll
    for (int db = 0; db < VP; ++db) {
      const int chunk = db * 4 + 2 * (g & 1) + ((s & 3) >> 1);
      voff[db] = St::V_BASE + vrow * St::ROW_BYTES + ((chunk ^ xv) << 4) + ((s & 1) << 3);
    }
  }

  // ---- this wave's share of every stage load (constant over the sweep) ------------------
  // A stage is WL 1-KiB loads of K rows followed by WL of V rows; load i = q*NW + wave is
  // this wave's q-th. Lane l of a load lands at byte 16*l of the load's LDS slot, which is
  // stage row j*RPL + l/CPR, physical chunk l%CPR; it fetches the row's logical chunk
  // (physical ^ swizzle) from global memory. The byte offset from the tensor base of the
  // stage depends only on the lane and q.
  const int64_t stage_stride = (int64_t)St::BKS * kv_row_stride;  // elements from one stage to the next
  const int64_t row_bytes_g = kv_row_stride * 2;                  // bytes between consecutive keys
  uint32_t dma_voff[St::LPW];  // per-lane byte offset of each load at stage 0
  int dma_row[St::LPW];        // its key row within a stage
  bool dma_isv[St::LPW];       // V (else K) load (wave-uniform)
  uint32_t dma_slot[St::LPW];  // LDS byte offset of the load within a stage (wave-uniform)
#pragma unroll
  for (int q = 0; q < St::LPW; ++q) {
    const int i = q * NW + wave;
    const bool isv = i >= St::WL;
    const int j = isv ? i - St::WL : i;
    const int row = j * St::RPL + lane / St::CPR;
    const int c = (lane % St::CPR) ^ (isv ? St::swz_v(row) : St::swz_k(row));
    dma_row[q] = row;
    dma_isv[q] = isv;
    dma_voff[q] = (uint32_t)(row * row_bytes_g + c * 16);
    dma_slot[q] = (isv ? St::V_BASE : 0) + j * 1024;
  }
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(tsp_lds_addr(smem));
  const float inv_scale_log2 = 1.0f / p.scale_log2;
  uint64_t ring_seen = 0;  // ring sweep: chunks (below 64) whose arrival flag this wave has seen set

  for (int which = 0; which < 2; ++which) {
    const int32_t qt = which == 0 ? p.n_qtiles - 1 - pair : pair;
    if (which == 1 && qt == p.n_qtiles - 1 - pair) break;  // middle tile of an odd count
    const int32_t row0 = qt * p.BQ;
    const int32_t last_row = min(row0 + p.BQ, p.S_local) - 1;
    const int32_t tile_end = tsp_zigzag_position(last_row, p.C, p.D, p.rank) + 1;  // keys the tile sees

    // ---- this wave's query rows -------------------------------------------------------
    int32_t lrow[RB], pos[RB], head[RB];
    bool rvalid[RB];
    int32_t wave_first = 0x7fffffff;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rbi = wave * RB + rb;
      const int pb = rbi % pos_blocks, hh = rbi / pos_blocks;
      head[rb] = hk * p.grp + hgrp * p.GH + hh;
      const int32_t r = row0 + pb * 32 + col;
      rvalid[rb] = r < p.S_local;
      lrow[rb] = min(r, p.S_local - 1);
      pos[rb] = tsp_zigzag_position(lrow[rb], p.C, p.D, p.rank);
      wave_first = min(wave_first, row0 + pb * 32);
    }
    const int32_t wave_min_pos = tsp_zigzag_position(min(wave_first, p.S_local - 1), p.C, p.D, p.rank);

    bool tile_sees = false;  // some key of the ranges is visible to some row of the tile
    // ring sweep: the chunk holding the tile's rows, and the number of peer chunks it sees
    const int32_t tile_chunk = row0 < p.C ? p.rank : 2 * p.D - 1 - p.rank;
    int32_t ring_n = 0;
    if constexpr (NR == 3) {
      for (int32_t s = 1; s < p.D; ++s) {
        const int32_t pp = (p.rank - s + p.D) % p.D;
        ring_n += (pp < tile_chunk) + (2 * p.D - 1 - pp < tile_chunk);
      }
      tile_sees = ring_n > 0;
    } else {
#pragma unroll
      for (int rg = 0; rg < NR; ++rg)
        tile_sees |= min(rg == 0 ? p.kv_hi : p.kv_hi2, tile_end) > (rg == 0 ? p.kv_lo : p.kv_lo2);
    }
    if (!tile_sees) {
      if (p.accumulate) continue;  // an empty partial leaves the running result as it is
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rvalid[rb]) {
          uint16_t* op = og + (((int64_t)b * p.S_local + lrow[rb]) * p.Hq + head[rb]) * DH + 4 * half;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) *reinterpret_cast<tsp_u32x2*>(op + db * 32 + 8 * a) = tsp_u32x2{0u, 0u};
          if (half == 0) p.lse[((int64_t)b * p.Hq + head[rb]) * p.S_local + lrow[rb]] = -INFINITY;
        }
      }
      continue;
    }

    // ---- Q^T operands stay in registers ------------------------------------------------
    tsp_bf16x8 qf[RB][NKK];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint16_t* qp = qg + (((int64_t)b * p.S_local + lrow[rb]) * p.Hq + head[rb]) * DH + half * 8;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qf[rb][kk] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(qp + kk * 16));
    }

    tsp_f32x16 acc[RB][NDB];
    float m_run[RB], l_run[RB];
    float m_thr[RB];  // a score above this (raw units) needs a higher running max
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = -INFINITY;
      m_thr[rb] = -INFINITY;
      l_run[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;
    }

    // ---- the keys of the sweep --------------------------------------------------------
    // The sweep starts at the stage boundary at or below kv_lo; key indices below are
    // relative to it (keys in [kv_base, kv_lo) are loaded but masked).
    const int32_t kv_base = NR == 3 ? 0 : (p.kv_lo / St::BKS) * St::BKS;
    const int32_t kv_lo_rel = NR == 3 ? 0 : p.kv_lo - kv_base;
    // relative end of the keys this tile sweeps: its last position, or the range end (the
    // ring sweep: its visible chunks back to back)
    const int32_t kv_end = NR == 3 ? ring_n * p.C : min(p.kv_hi, tile_end) - kv_base;
    const uint16_t* __restrict__ kbase = kg + ((int64_t)b * p.S_total + kv_base) * p.kv_stride + (int64_t)hk * DH;
    const uint16_t* __restrict__ vbase = vg + ((int64_t)b * p.S_total + kv_base) * p.kv_stride + (int64_t)hk * DH;
    int32_t n_kv1 = (kv_end + BK - 1) / BK;             // pipeline steps
    int32_t n_stage1 = (kv_end + St::BKS - 1) / St::BKS;  // stages
    // last visible key of each row: its position, or the range end if that comes first
    int32_t qpos[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) qpos[rb] = min(pos[rb], p.kv_hi - 1);
    // steps [u_left, t_mask) are visible to every row of the wave; earlier steps hold keys
    // below kv_lo, later ones keys past some row's position or the range end: all masked
    // (the ring sweep has no masked step)
    int32_t t_mask = NR == 3 ? n_kv1 : min(n_kv1, max(0, min(wave_min_pos + 1, p.kv_hi) - kv_base) / BK);
    const int32_t u_left = (kv_lo_rel + BK - 1) / BK;
    // The second range (two-range launches): its stages follow the first range's whole
    // stages in the ring and its steps start at step T1; its keys are indexed from its own
    // stage-aligned start kv_base2. A tile that sees a key of it also sees the first range,
    // which lies below (an unseen first range is dropped all the same).
    int32_t T1 = n_kv1, n_kv2 = 0, n_stage2 = 0;
    int32_t kv_base2 = 0, kv_lo_rel2 = 0, kv_end2 = 0, t_mask2 = 0, u_left2 = 0;
    int32_t qpos2[RB];
    const uint16_t* __restrict__ kbase2 = kbase;
    const uint16_t* __restrict__ vbase2 = vbase;
    bool run_on = false;  // the unmasked steps run on from the first range into the second
    if constexpr (NR == 2) {
      int32_t n_full1 = kv_end / St::BKS;
      if (kv_end <= kv_lo_rel) n_kv1 = n_stage1 = t_mask = n_full1 = T1 = 0;
      kv_base2 = (p.kv_lo2 / St::BKS) * St::BKS;
      kv_lo_rel2 = p.kv_lo2 - kv_base2;
      kv_end2 = min(p.kv_hi2, tile_end) - kv_base2;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) qpos2[rb] = min(pos[rb], p.kv_hi2 - 1);
      if (kv_end2 > kv_lo_rel2) {
        T1 = n_stage1 * SPS;  // the first range's steps, padded to whole stages
        n_kv2 = (kv_end2 + BK - 1) / BK;
        n_stage2 = (kv_end2 + St::BKS - 1) / St::BKS;
        t_mask2 = min(n_kv2, max(0, min(wave_min_pos + 1, p.kv_hi2) - kv_base2) / BK);
        u_left2 = (kv_lo_rel2 + BK - 1) / BK;
        kbase2 = kg + ((int64_t)b * p.S_total + kv_base2) * p.kv_stride + (int64_t)hk * DH;
        vbase2 = vg + ((int64_t)b * p.S_total + kv_base2) * p.kv_stride + (int64_t)hk * DH;
        run_on = n_full1 == n_stage1 && t_mask == T1 && u_left2 == 0;
      }
    }
    const int64_t stage_off2 = (int64_t)n_stage1 * stage_stride;  // offset of the second range's stages
    const int32_t n_kv = T1 + n_kv2;              // pipeline steps of both ranges
    const int32_t n_stage = n_stage1 + n_stage2;  // stages of both ranges

    // ---- ring sweep: physical first key of virtual stage sg ------------------------------
    // Stages are asked for in order, each once; the cursor moves to the next visible chunk
    // at a chunk's first stage. The chunk's arrival is checked beforehand by ring_poll_upto.
    constexpr int32_t RING_E_MAX = 1 << 20;
    auto ring_advance = [&](int32_t& e) -> int32_t {  // next visible chunk after ring index e
      const int32_t n_e = min(2 * (p.D - 1), RING_E_MAX);
      int32_t c = 0;
      do {
        ++e;
        const int32_t pp = (p.rank - (1 + e / 2) + p.D) % p.D;
        c = (e & 1) ? 2 * p.D - 1 - pp : pp;
      } while (c >= tile_chunk && e < n_e);
      return c >= tile_chunk ? 0 : c;  // 0 not reached: the count of visible chunks bounds the calls
    };
    int32_t ring_e = -1, ring_chunk = 0, ring_next = 0;  // load cursor: ring index, chunk, next chunk's first stage
    auto ring_stage_key = [&](int32_t sg) -> int32_t {
      const int32_t spc = p.C / St::BKS;  // stages per chunk
      if (sg == ring_next) {
        ring_chunk = ring_advance(ring_e);
        ring_next += spc;
      }
      return ring_chunk * p.C + (sg - (ring_next - spc)) * St::BKS;
    };
    // Arrival: before any stage up to sg_max is loaded, wait (bounded) for the chunks those
    // stages start. Wave 0 alone reads the flags (the acquire invalidates the caches, which
    // is costly when every wave does it), then a workgroup barrier orders every wave's
    // stage loads after that acquire. A flag load also drains wave 0's in-flight stage
    // loads (the compiler waits for every vector load before using its value), so this runs
    // outside the unrolled steps, reads both chunks of a ring step at once, and skips chunks
    // already seen present (also for the pair's other tile). Every wave takes the barrier
    // at the same points: the chunk cursor is the same in all of them.
    int32_t poll_e = -1, poll_next = 0, poll_done = 0;
    auto ring_poll_upto = [&](int32_t sg_max) {
      if (p.ready == nullptr) return;
      const int32_t spc = p.C / St::BKS;
      bool polled = false;
      while (poll_next <= sg_max && poll_done < ring_n) {
        const int32_t c = ring_advance(poll_e);
        poll_next += spc;
        ++poll_done;
        polled = true;
        if (wave != 0 || (c < 64 && ((ring_seen >> c) & 1))) continue;
        const int32_t pp = (p.rank - (1 + poll_e / 2) + p.D) % p.D;
        const int32_t ca = pp, cb = 2 * p.D - 1 - pp;  // the ring step's two chunks
        bool arrived = false;
        for (int32_t it = 0; it < p.spin_limit && !arrived; ++it) {
          const int32_t fa = __hip_atomic_load(p.ready + ca, __ATOMIC_ACQUIRE, TSP_RING_SCOPE);
          const int32_t fb = __hip_atomic_load(p.ready + cb, __ATOMIC_ACQUIRE, TSP_RING_SCOPE);
          const bool ra = __builtin_amdgcn_readfirstlane(fa) == p.ready_value;
          const bool rb = __builtin_amdgcn_readfirstlane(fb) == p.ready_value;
          if (ra && ca < 64) ring_seen |= uint64_t(1) << ca;
          if (rb && cb < 64) ring_seen |= uint64_t(1) << cb;
          arrived = c == ca ? ra : rb;
          if (!arrived) __builtin_amdgcn_s_sleep(2);
        }
        if (!arrived && lane == 0) atomicOr(p.wait_status, 1);
      }
      if (polled) __syncthreads();
    };

    // ---- stage loads: global -> LDS, this wave's share --------------------------------
    // Any stage: rows past the tile's last position (or its range's end) are clamped to it
    // (never read past it).
    auto issue_stage = [&](int s) {
      const uint16_t* kb = kbase;
      const uint16_t* vb = vbase;
      int32_t kv0 = s * St::BKS, end = kv_end;
      if constexpr (NR == 3) {  // a whole stage of a visible chunk
        ring_poll_upto(s);
        const int32_t k0 = ring_stage_key(s);
        const uint32_t base = smem_addr + (s % NBUF) * St::SLOT_STRIDE;
#pragma unroll
        for (int q = 0; q < St::LPW; ++q)
          tsp_lds_dma16((dma_isv[q] ? vb : kb) + (int64_t)k0 * kv_row_stride, dma_voff[q], base + dma_slot[q]);
        return;
      }
      if constexpr (NR == 2) {
        if (s >= n_stage1) {  // a stage of the second range
          kb = kbase2;
          vb = vbase2;
          kv0 = (s - n_stage1) * St::BKS;
          end = kv_end2;
        }
      }
      const uint32_t base = smem_addr + (s % NBUF) * St::SLOT_STRIDE;
#pragma unroll
      for (int q = 0; q < St::LPW; ++q) {
        const int32_t over = max(0, kv0 + dma_row[q] - (end - 1));  // rows beyond the last key
        const uint16_t* tb = (dma_isv[q] ? vb : kb) + (int64_t)kv0 * kv_row_stride;
        tsp_lds_dma16(tb, dma_voff[q] - (uint32_t)(over * row_bytes_g), base + dma_slot[q]);
      }
    };
    // Wait until stage s has landed for every wave; the stages issued after it (up to
    // last_issued) stay in flight.
    auto stage_ready = [&](int s, int last_issued) {
      tsp_wait_vmcnt(St::LPW * (last_issued - s));
      __syncthreads();
    };

    // ---- pipeline pieces ---------------------------------------------------------------
    // step t reads keys [32t, 32t+32): stage t/SPS, rows 32*(t%SPS) .. of its slot
    auto qk = [&](int t, tsp_f32x16(&sc)[RB]) {
      const uint8_t* kt = smem + ((t / SPS) % NBUF) * St::SLOT_STRIDE + (t % SPS) * BK * St::ROW_BYTES;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[rb][e] = 0.f;
      tsp_bf16x8 kf[NKK];  // all K operands of the step in flight before the first MFMA
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kf[kk] = __builtin_bit_cast(tsp_bf16x8,
                                    *reinterpret_cast<const tsp_u32x4*>(kt + koff[kk % KP] + (kk / KP) * St::SWZ * 16));
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[rb][kk], sc[rb], 0, 0, 0);
    };
    // key kv_base + s*BK + 8(e/4) + 4*half + (e%4) of query column `col` is visible iff
    // it is <= qpos (the query's position, capped below kv_hi) and >= kv_lo; in the second
    // range, key kv_base2 + (s - T1)*BK + ... against qpos2 and kv_lo2
    auto mask = [&](int s, tsp_f32x16(&sc)[RB]) {
      int32_t lo_rel = kv_lo_rel, base = kv_base, u = s;
      bool second = false;
      if constexpr (NR == 2) {
        second = s >= T1;
        if (second) {
          lo_rel = kv_lo_rel2;
          base = kv_base2;
          u = s - T1;
        }
      }
      const int32_t lo = lo_rel - u * BK - 4 * half;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        int32_t last = qpos[rb];
        if constexpr (NR == 2) last = second ? qpos2[rb] : last;
        const int32_t hi = last - base - u * BK - 4 * half;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = 8 * (e >> 2) + (e & 3);
          if (off > hi || off < lo) sc[rb][e] = -INFINITY;
        }
      }
    };
    auto needs_mask = [&](int s) {
      if constexpr (NR == 2) {
        if (s >= T1) return s - T1 >= t_mask2 || s - T1 < u_left2;
      }
      return s >= t_mask || s < u_left;
    };
    // Row max of a step's scores over this lane's 16 keys (raw score units): the two
    // halves of a row are tested separately, which decides the same wave-wide ballot as
    // testing the full row, and the full max is formed only when a rescale is due.
    auto rowmax = [&](const tsp_f32x16(&sc)[RB], float(&mx)[RB]) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float m = sc[rb][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) m = fmaxf(m, sc[rb][e]);
        mx[rb] = m;
      }
    };
    auto rescale_needed = [&](const float(&mx)[RB]) {
      bool need = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) need |= mx[rb] > m_thr[rb];
      return __builtin_amdgcn_ballot_w64(need) != 0;  // wave-uniform
    };
    // Raise the running max to cover this step (rare after the first step): scale the
    // accumulated output and sum by 2^(m_old - m_new).
    auto rescale = [&](const float(&mx)[RB]) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_new = fmaxf(m_run[rb], tsp_max_halves(mx[rb]) * p.scale_log2);
        m_thr[rb] = (m_new + TSP_RESCALE_SLACK) * inv_scale_log2;
        // a row with no visible key yet (both -inf) keeps its zero state
        const float alpha = m_new == -INFINITY ? 1.f : tsp_exp2(m_run[rb] - m_new);
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[rb][db][e] *= alpha;
      }
    };
    // guard: a row may not have seen a visible key yet (m_run = -inf), so use 0 as its
    // exponent offset; its scores are all -inf and its weights 0
    auto softmax = [&](const tsp_f32x16(&sc)[RB], tsp_bf16x8(&pf)[RB][2], bool guard) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mneg = (guard && m_run[rb] == -INFINITY) ? 0.f : -m_run[rb];
        float lsum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float pw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pw[e] = tsp_exp2(fmaf(sc[rb][st * 8 + e], p.scale_log2, mneg));
          tsp_u32x4 w;
          w[0] = tsp_pack_bf16(pw[0], pw[1]);
          w[1] = tsp_pack_bf16(pw[2], pw[3]);
          w[2] = tsp_pack_bf16(pw[4], pw[5]);
          w[3] = tsp_pack_bf16(pw[6], pw[7]);
          // the row sum uses the rounded weights the PV product applies
#pragma unroll
          for (int e = 0; e < 4; ++e) lsum = tsp_sum_bf16_pair(w[e], lsum);
          pf[rb][st] = __builtin_bit_cast(tsp_bf16x8, w);
        }
        l_run[rb] += lsum;
      }
    };
    auto pv = [&](int t, const tsp_bf16x8(&pf)[RB][2]) {
      const uint8_t* vt =
          smem + ((t / SPS) % NBUF) * St::SLOT_STRIDE + (t % SPS) * BK * St::ROW_BYTES;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint8_t* a = vt + voff[db % VP] + (db / VP) * St::SWZ * 16 + st * 16 * St::ROW_BYTES;
          const tsp_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a));
          const tsp_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a + 8 * St::ROW_BYTES));
          const tsp_bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb][st], acc[rb][db], 0, 0, 0);
        }
      }
    };

    for (int attempt = 0;; ++attempt) {  // a second sweep only after an overflow (FIXED_MAX)
      if (attempt > 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          m_run[rb] = -INFINITY;
          m_thr[rb] = -INFINITY;
          l_run[rb] = 0.f;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;
        }
      }
      // ---- prologue -------------------------------------------------------------------
      __syncthreads();  // the previous tile's readers are done with every buffer
      const int pro = min(PD, n_stage - 1);
      for (int s = 0; s <= pro; ++s) issue_stage(s);
      stage_ready(0, pro);

      tsp_f32x16 s_cur[RB];
      float mx[RB];
      qk(0, s_cur);
      if (needs_mask(0)) mask(0, s_cur);
      rowmax(s_cur, mx);
      if constexpr (FIXED_MAX) {
        if (rescale_needed(mx)) rescale(mx);  // the running max the unrolled steps keep
      }

      // ---- main sweep ----------------------------------------------------------------------
      // Fast path: steps whose successor needs no mask and whose prefetched stage lies fully
      // below the end of its range. Unrolled over whole ring cycles so every LDS slot is a compile-time
      // offset and the two score tiles alternate without copies; constant vmcnt; no clamping.
      constexpr int VM_STEADY = St::LPW * (PD - 1);
      static_assert(VM_STEADY < 16, "vmcnt immediate");
      constexpr int GROUP = (NBUF * SPS) % 2 == 0 ? NBUF * SPS : 2 * NBUF * SPS;  // steps per unrolled group
      int32_t n_full = kv_end / St::BKS;  // stages with every key below the end of their range
      int32_t t_unmasked = t_mask;        // the steps from u_left up to it need no mask
      if constexpr (NR == 2) {
        if (run_on) {
          n_full = n_stage1 + kv_end2 / St::BKS;
          t_unmasked = T1 + t_mask2;
        }
      }
      const int t_fast = u_left == 0 && attempt == 0 ? min(t_unmasked - 1, (n_full - PD) * SPS - 1) : 0;
      tsp_f32x16 s_alt[RB];
      // Stage boundary: wait until stage NEXT (relative to t0 / SPS) landed for every wave,
      // then issue the stage PD ahead into the slot two stages back.
      auto boundary = [&](auto next_const, int t0) {
        constexpr int NEXT = decltype(next_const)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | VM_STEADY);  // that stage landed (this wave's part)
        __syncthreads();  // ... for every wave; the slot two stages back is free again
        const int32_t sg = t0 / SPS + NEXT + PD;  // the stage to issue
        int64_t adv = (int64_t)sg * stage_stride;
        if constexpr (NR == 3) adv = (int64_t)ring_stage_key(sg) * kv_row_stride;
        const uint16_t* kb = kbase;
        const uint16_t* vb = vbase;
        if constexpr (NR == 2) {
          if (sg >= n_stage1) {  // a stage of the second range
            kb = kbase2;
            vb = vbase2;
            adv -= stage_off2;
          }
        }
        const uint32_t base = smem_addr + ((NEXT + PD) % NBUF) * St::SLOT_STRIDE;
#pragma unroll
        for (int q = 0; q < St::LPW; ++q)
          tsp_lds_dma16((dma_isv[q] ? vb : kb) + adv, dma_voff[q], base + dma_slot[q]);
      };
      // LAG (second half of the waves, one of the two waves of each SIMD): the barrier of
      // stage k comes after the PV products of step SPS*k - 2 instead of before the QK
      // products of step SPS*k - 1. Every barrier still precedes the first read of its stage
      // and follows the last read of the stage two back, but the two waves of a SIMD then run
      // their matrix and vector phases in alternation (one's softmax under the other's MFMAs).
      auto fast_step = [&](auto u_const, auto lag_const, int t0) {
        constexpr int U = decltype(u_const)::value;  // step t = t0 + U, t0 a multiple of GROUP
        constexpr bool LAG = decltype(lag_const)::value;
        tsp_f32x16(&sc)[RB] = (U % 2 == 0) ? s_cur : s_alt;
        tsp_f32x16(&sn)[RB] = (U % 2 == 0) ? s_alt : s_cur;
        if constexpr (!FIXED_MAX) {
          if (rescale_needed(mx)) rescale(mx);
        }
        if constexpr (!LAG && (U + 1) % SPS == 0)  // step t+1 opens a new stage
          boundary(std::integral_constant<int, (U + 1) / SPS>{}, t0);
        tsp_bf16x8 pf[RB][2];
        qk(U + 1, sn);     // matrix pipe: next step's scores
        softmax(sc, pf, false);  // vector pipe: this step's weights
        pv(U, pf);         // matrix pipe: this step's output
        if constexpr (LAG && (U + 2) % SPS == 0)  // the next stage's barrier, one phase early
          boundary(std::integral_constant<int, (U + 2) / SPS>{}, t0);
        if constexpr (!FIXED_MAX) rowmax(sn, mx);  // vector pipe: next step's row max
      };
      auto fast_group = [&]<int... Us>(std::integer_sequence<int, Us...>, auto lag_const, int t0) {
        (fast_step(std::integral_constant<int, Us>{}, lag_const, t0), ...);
      };
      // PINNED (one wave per SIMD, one step per stage): each step in a fixed issue order,
      // since no second wave covers this wave's waits. Phase A: the 16 QK^T products of step
      // t+1, each K operand read KW operands ahead of its products, and under each product
      // an equal share of the V^T operand reads and of the weights of step t. Phase B: the
      // 16 PV products of step t back to back; after product BJ, the stage boundary (stage
      // t+2 landed, barrier), then the first KW K operands of step t+2 and the load of stage
      // t+4 into the slot of stage t, whose reads all ended before the barrier.
      constexpr bool PINNED = FIXED_MAX && SPS == 1 && TSP_FWD_PINNED;
      constexpr int KW = TSP_PIN_KW > 0 ? TSP_PIN_KW : RB == 1 ? 4 : 2, BJ = TSP_PIN_BJ;
      constexpr int NOPS = KW + St::LPW, PER = (NOPS + 14 - BJ) / (15 - BJ);  // ops per PV product after the barrier
      static_assert(!PINNED || (NBUF == 4 && NKK * RB == 16 && 2 * NDB * RB == 16), "16 + 16 products a step, 4 slots");
      tsp_bf16x8 kw[KW];  // the first K operands of the next step's QK^T products
      // SPLIT (two row blocks): row block 0's weights of step t+1 are computed under the PV
      // products of step t, so each product of both phases carries one weight
      constexpr bool SPLIT = PINNED && RB == 2 && TSP_PIN_SPLIT;
      tsp_u32x4 wc[2];  // SPLIT: row block 0's rounded weights of the next step
      float lc = 0.f;   // ... and their sum
      // weight e (0..15) of a row: 2^(score * scale - m), rounded to bf16 in pairs; the row
      // sum takes the rounded pairs, as PV applies them
      auto weight = [&](float score, float mn, float(&pwr)[16], tsp_u32x4(&wr)[2], float& ls, int e,
                        bool here = false) {
        pwr[e] = tsp_exp2(fmaf(score, p.scale_log2, mn));
        if (here) asm volatile("" : "+v"(pwr[e]));  // computed at this point of the order, not where used
        if (e & 1) {
          wr[e / 8][(e % 8) / 2] = tsp_pack_bf16(pwr[e - 1], pwr[e]);
          ls = tsp_sum_bf16_pair(wr[e / 8][(e % 8) / 2], ls);
          if (here) asm volatile("" : "+v"(ls));
        }
      };
      auto kread = [&](const uint8_t* kt, int kk) {
        return __builtin_bit_cast(tsp_bf16x8,
                                  *reinterpret_cast<const tsp_u32x4*>(kt + koff[kk % KP] + (kk / KP) * St::SWZ * 16));
      };
      auto vread = [&](const uint8_t* vt, int j) {  // PV operand j: st = j / NDB, db = j % NDB
        const uint8_t* a = vt + voff[(j % NDB) % VP] + ((j % NDB) / VP) * St::SWZ * 16 + (j / NDB) * 16 * St::ROW_BYTES;
        const tsp_bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a));
        const tsp_bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a + 8 * St::ROW_BYTES));
        return tsp_bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      auto pinned_step = [&](auto u_const, int t0) {
        constexpr int U = decltype(u_const)::value;  // step t = t0 + U, t0 a multiple of NBUF
        constexpr int NV = 2 * NDB;                   // V^T operands of a step
        tsp_f32x16(&sc)[RB] = (U % 2 == 0) ? s_cur : s_alt;
        tsp_f32x16(&sn)[RB] = (U % 2 == 0) ? s_alt : s_cur;
        const uint8_t* kt = smem + ((U + 1) % NBUF) * St::SLOT_STRIDE;  // K of step t+1
        const uint8_t* vt = smem + (U % NBUF) * St::SLOT_STRIDE;        // V of step t
        const uint8_t* kt2 = smem + ((U + 2) % NBUF) * St::SLOT_STRIDE;  // K of step t+2
        tsp_bf16x8 kf[NKK], vf[NV];
        float pw[RB][16], lsum[RB], mneg[RB];
        tsp_u32x4 w[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          lsum[rb] = 0.f;
          mneg[rb] = -m_run[rb];
#pragma unroll
          for (int e = 0; e < 16; ++e) sn[rb][e] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < KW; ++j) kf[j] = kw[j];
#pragma unroll
        for (int j = 0; j < 16; ++j) {  // phase A: product j is (K operand j / RB, row block j % RB)
          const int kk = j / RB, rq = j % RB;
          sn[rq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[rq][kk], sn[rq], 0, 0, 0);
          if (rq == 0 && kk + KW < NKK) kf[kk + KW] = kread(kt, kk + KW);
#pragma unroll
          for (int o = j * NV / 16; o < (j + 1) * NV / 16; ++o) vf[o] = vread(vt, o);
          if constexpr (SPLIT) {
            weight(sc[1][j], mneg[1], pw[1], w[1], lsum[1], j);
          } else {
#pragma unroll
            for (int x = j * RB; x < (j + 1) * RB; ++x)  // weight x: row block x / 16, score x % 16
              weight(sc[x / 16][x % 16], mneg[x / 16], pw[x / 16], w[x / 16], lsum[x / 16], x % 16);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        tsp_bf16x8 pf[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bool carried = SPLIT && rb == 0;
          l_run[rb] += carried ? lc : lsum[rb];
          pf[rb][0] = __builtin_bit_cast(tsp_bf16x8, carried ? wc[0] : w[rb][0]);
          pf[rb][1] = __builtin_bit_cast(tsp_bf16x8, carried ? wc[1] : w[rb][1]);
        }
        // the load of stage t+4 (a stage of the second range past the first's stages)
        const int32_t sg = t0 + U + 4;
        int64_t adv = (int64_t)sg * stage_stride;
        const uint16_t* kb = kbase;
        const uint16_t* vb = vbase;
        if constexpr (NR == 2) {
          if (sg >= n_stage1) {
            kb = kbase2;
            vb = vbase2;
            adv -= stage_off2;
          }
        }
        const uint32_t base = smem_addr + ((U + 4) % NBUF) * St::SLOT_STRIDE;
#pragma unroll
        for (int j = 0; j < 16; ++j) {  // phase B: product j is (V^T operand j / RB, row block j % RB)
          const int o = j / RB, rq = j % RB;
          acc[rq][o % NDB] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[o], pf[rq][o / NDB], acc[rq][o % NDB], 0, 0, 0);
          if (j == BJ) {
            __builtin_amdgcn_s_waitcnt(0x0F70 | VM_STEADY);  // stage t+2 landed (this wave's part)
            __syncthreads();  // ... for every wave; every read of stage t is done
          }
          if (j > BJ) {
#pragma unroll
            for (int o = (j - BJ - 1) * PER; o < (j - BJ) * PER && o < NOPS; ++o) {
              if (o < KW) {
                kw[o] = kread(kt2, o);
              } else {
                const int q = o - KW;
                tsp_lds_dma16((dma_isv[q] ? vb : kb) + adv, dma_voff[q], base + dma_slot[q]);
              }
            }
          }
          if constexpr (SPLIT) weight(sn[0][j], mneg[0], pw[0], w[0], lsum[0], j, true);  // step t+1
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SPLIT) {
          wc[0] = w[0][0];
          wc[1] = w[0][1];
          lc = lsum[0];
        }
      };
      auto pinned_group = [&]<int... Us>(std::integer_sequence<int, Us...>, int t0) {
        (pinned_step(std::integral_constant<int, Us>{}, t0), ...);
      };
      int t = 0;
      constexpr bool PINGPONG = TSP_PINGPONG && SPS == 2 && NW % 2 == 0;
      if constexpr (PINNED) {
        // one stage less ahead: the last pinned step loads stage t+4
        const int t_pin = min(t_fast, (n_full - PD - 1) * SPS - 1);
        if (t_pin >= GROUP) {
          boundary(std::integral_constant<int, 1>{}, 0);  // stage 1 ready; stage 3 issued
#pragma unroll
          for (int j = 0; j < KW; ++j) kw[j] = kread(smem + 1 * St::SLOT_STRIDE, j);
          if constexpr (SPLIT) {  // row block 0's weights of the first pinned step
            float pw0[16];
            lc = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) weight(s_cur[0][e], -m_run[0], pw0, wc, lc, e);
          }
          for (; t + GROUP <= t_pin; t += GROUP) pinned_group(std::make_integer_sequence<int, GROUP>{}, t);
        }
      } else if (PINGPONG && TSP_PP_LAGGED(wave)) {
        for (; t + GROUP <= t_fast; t += GROUP) {
          if constexpr (NR == 3) ring_poll_upto(t / SPS + PD + GROUP / SPS);  // the stages this group loads
          fast_group(std::make_integer_sequence<int, GROUP>{}, std::bool_constant<PINGPONG>{}, t);
        }
      } else {
        for (; t + GROUP <= t_fast; t += GROUP) {
          if constexpr (NR == 3) ring_poll_upto(t / SPS + PD + GROUP / SPS);
          fast_group(std::make_integer_sequence<int, GROUP>{}, std::false_type{}, t);
        }
      }
      if constexpr (FIXED_MAX) {
        if (t > 0) rowmax(s_cur, mx);  // the next step's scores (GROUP is even)
      }
      int issued = t > 0 ? t / SPS + PD + (PINNED ? 1 : 0) : pro;  // last stage issued so far
      // PINNED: the last stage already waited for (and barriered) by the pinned steps. Every
      // wave takes barrier k when stage k+1 is ready and then loads stage k+3, on either path.
      const int ready = PINNED && t > 0 ? t + 1 : 0;

      // General path: the masked steps near the diagonal, the partial last stage and the
      // ring drain.
      for (; t < n_kv; ++t) {
        if (rescale_needed(mx)) rescale(mx);
        tsp_bf16x8 pf[RB][2];
        if (t + 1 < n_kv) {
          if ((t + 1) % SPS == 0 && (!PINNED || (t + 1) / SPS > ready)) {
            stage_ready((t + 1) / SPS, issued);
            if (issued + 1 < n_stage) issue_stage(++issued);
          }
          qk(t + 1, s_alt);
          softmax(s_cur, pf, true);
          pv(t, pf);
          if (needs_mask(t + 1)) mask(t + 1, s_alt);
          rowmax(s_alt, mx);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s_cur[rb] = s_alt[rb];
        } else {
          softmax(s_cur, pf, true);
          pv(t, pf);
        }
      }
      if constexpr (!FIXED_MAX) break;
      if (attempt > 0) break;
      // an infinite or NaN sum or output (exponent field all ones) anywhere in the workgroup
      uint32_t top = 0;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        top = max(top, __float_as_uint(l_run[rb]) & 0x7fffffffu);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) top = max(top, __float_as_uint(acc[rb][db][e]) & 0x7fffffffu);
      }
      if (!__syncthreads_or(top >= 0x7f800000u)) break;
    }  // attempt

    // ---- epilogue: normalise, round to bf16, write O and lse -----------------------------
    if (p.accumulate) {  // merge this partial into the running result (out, lse)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l = tsp_sum_halves(l_run[rb]);
        if (!rvalid[rb] || !(l > 0.f)) continue;  // no visible key: nothing to add
        float* lp = p.lse + ((int64_t)b * p.Hq + head[rb]) * p.S_local + lrow[rb];
        float w_old, w_new;
        const float lse_new = tsp_merge_weights(*lp, m_run[rb], l, w_old, w_new);
        uint16_t* op = og + (((int64_t)b * p.S_local + lrow[rb]) * p.Hq + head[rb]) * DH + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            tsp_u32x2* dst = reinterpret_cast<tsp_u32x2*>(op + db * 32 + 8 * a);
            const tsp_u32x2 o = *dst;
            tsp_u32x2 w;
            w[0] = tsp_pack_bf16(fmaf(w_new, acc[rb][db][4 * a + 0], w_old * __uint_as_float(o[0] << 16)),
                                 fmaf(w_new, acc[rb][db][4 * a + 1], w_old * __uint_as_float(o[0] & 0xffff0000u)));
            w[1] = tsp_pack_bf16(fmaf(w_new, acc[rb][db][4 * a + 2], w_old * __uint_as_float(o[1] << 16)),
                                 fmaf(w_new, acc[rb][db][4 * a + 3], w_old * __uint_as_float(o[1] & 0xffff0000u)));
            *dst = w;
          }
        // both halves of the wave have read the old lse above (the weights depend on it)
        if (half == 0) *lp = lse_new;
      }
      continue;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l = tsp_sum_halves(l_run[rb]);
      const float inv = l > 0.f ? 1.0f / l : 0.f;  // l = 0: no visible key in the range
      if (rvalid[rb]) {
        uint16_t* op = og + (((int64_t)b * p.S_local + lrow[rb]) * p.Hq + head[rb]) * DH + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            tsp_u32x2 w;
            w[0] = tsp_pack_bf16(acc[rb][db][4 * a + 0] * inv, acc[rb][db][4 * a + 1] * inv);
            w[1] = tsp_pack_bf16(acc[rb][db][4 * a + 2] * inv, acc[rb][db][4 * a + 3] * inv);
            *reinterpret_cast<tsp_u32x2*>(op + db * 32 + 8 * a) = w;
          }
        if (half == 0)
          p.lse[((int64_t)b * p.Hq + head[rb]) * p.S_local + lrow[rb]] =
              l > 0.f ? (m_run[rb] + __builtin_amdgcn_logf(l)) * TSP_LN2 : -INFINITY;
      }
    }
  }
}

}  // namespace tsp
