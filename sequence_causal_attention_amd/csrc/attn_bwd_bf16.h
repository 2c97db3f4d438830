// attn_bwd_bf16.h -- backward of the per-rank causal attention, bf16 in, fp32 accumulation,
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) for every product.
//
// What is computed: the gradient of the forward (attn_fwd_bf16.h) for an upstream
// gradient dO of out. The pages describe training systems ("Folding Tensor and Sequence
// Parallelism for Memory-Efficient Transformer Training & Inference"; "AutoSP ...",
// section 2.B: attention is recomputed in the backward pass); the gradient follows from
// the chain rule through the softmax. With P_ij = exp(s_ij - lse_i) on visible pairs,
// s_ij = q_i . k_j / sqrt(dh), and Delta_i = dO_i . O_i (= sum_j P_ij dP_ij):
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - Delta_i),
//   dQ_i = sum_j dS_ij k_j / sqrt(dh),   dK_j = sum_i dS_ij q_i / sqrt(dh).
// dK / dV are the rank's partial gradients of the gathered K/V (summed over the query
// heads of each KV head); the adjoint of the K/V all-gather adds the ranks' partials.
//
// Three kernels, no atomics and no scratch buffer:
//  * attn_bwd_delta_kernel: Delta_i, one fp32 per (row, head) from the bf16 O and dO.
//  * attn_bwd_dkv_bf16_kernel (key-stationary): a workgroup owns 32*NW keys of one KV
//    head, each wave 32 of them, with its K and V rows as MFMA B operands in registers
//    (or, in the one-launch form at dh <= 128, its V rows parked in LDS). It sweeps the 32-row tiles of Q and dO (every query head of the group, every tile
//    whose rows see the keys) through an LDS ring. Scores are computed as S = Q K^T, with
//    queries on MFMA rows and keys on columns: each lane holds one key, so P and dS,
//    rounded to bf16, are directly the B operands of dV^T += dO^T P and dK^T += Q^T dS,
//    whose A operands come from the same LDS tiles through the transposing read
//    ds_read_b64_tr_b16. The GQA sum over query heads stays in the accumulators.
//  * attn_bwd_dq_bf16_kernel (query-stationary, the forward's decomposition): scores
//    transposed, S^T = K Q^T and dP^T = V dO^T, with Q^T and dO^T in registers; dS^T is
//    the B operand of dQ^T += K^T dS^T, K^T read transposed from the K tile.
//  The Q, dO (dK/dV kernel) and K (dQ kernel) tiles are read both row-wise and through
//  the transposing read; their 16-byte chunks are XOR-swizzled with
//  f(row) = 4*(row%4) + (row/4)%4, which keeps both patterns free of bank conflicts:
//  16 consecutive rows at one chunk land on 16 distinct chunks, and the 4 rows x 2
//  chunks of one 16-lane transposing group on 8 distinct chunk slots.
#pragma once

#include "attn_common.h"
#include "attn_fwd_bf16.h"

#ifndef TSP_BWD_UNROLL_RING_PIPE
#define TSP_BWD_UNROLL_RING_PIPE 1
#endif
#ifndef TSP_BWD_UNROLL_RING_NOPIPE
#define TSP_BWD_UNROLL_RING_NOPIPE 1
#endif
#ifndef TSP_BWD_READ_AHEAD
#define TSP_BWD_READ_AHEAD 1
#endif

namespace tsp {

typedef float tsp_f32x4 __attribute__((ext_vector_type(4)));

struct TspBwdParams {
  TspParams f;          // q, k, v, out, lse and the query-tile plan of the dQ kernel
  const void* dout;     // [B, S_local, Hq, dh]
  void* dq;             // [B, S_local, Hq, dh]
  void* dk;             // [B, S_total, Hkv, dh]
  void* dv;             // [B, S_total, Hkv, dh]
  float* delta;         // [B, Hq, S_local]
  int64_t n_rows;       // B * S_local * Hq
  int64_t n_kv_rows;    // B * S_total * Hkv
  int32_t kv_need;      // (2D - rank) * C: keys that some local row sees
  int32_t n_kblocks;    // key blocks of the dK/dV kernel per (b, KV head)
  float scale;          // 1 / sqrt(dh)
};

// 4 bytes per lane from global memory straight into LDS: lane i reads *gaddr and writes
// lds_addr + 4*i (global_load_lds_dword, address form, LDS base in M0).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void tsp_lds_dma4(const void* gaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gaddr), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Chunk swizzle of a tile read both row-wise and transposed (see the header comment).
template <int CPR>
__device__ __forceinline__ int tsp_swz_rt(int row) {
  if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (row >> 1) & 7;  // 128-byte rows: two rows per bank line
}

// Byte offsets of the transposing read of a swizzled tile: the A operand of a
// [32 dims x 16 rows] block db, rows 4*half + {0..3} (lo) and 8 + 4*half + {0..3} (hi),
// in each 16-lane group g lane s addressing row +s/4 and dims db*32 + 16(g&1) + 4(s&3).
template <int DH>
__device__ __forceinline__ void tsp_tr_offsets(int lane, int (&lo)[DH / 32], int (&hi)[DH / 32]) {
  constexpr int CPR = DH / 8, RB = DH * 2;
  const int half = lane >> 5, g = lane >> 4, s = lane & 15;
  const int r0 = 4 * half + (s >> 2), r1 = r0 + 8;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) {
    const int chunk = db * 4 + 2 * (g & 1) + ((s & 3) >> 1);
    lo[db] = r0 * RB + ((chunk ^ tsp_swz_rt<CPR>(r0)) << 4) + ((s & 1) << 3);
    hi[db] = r1 * RB + ((chunk ^ tsp_swz_rt<CPR>(r1)) << 4) + ((s & 1) << 3);
  }
}

__device__ __forceinline__ tsp_bf16x8 tsp_tr_read8(const uint8_t* lo, const uint8_t* hi) {
  const tsp_bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(lo));
  const tsp_bf16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(hi));
  return tsp_bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
}

__device__ __forceinline__ tsp_bf16x8 tsp_pack8(const float* x) {
  tsp_u32x4 w;
  w[0] = tsp_pack_bf16(x[0], x[1]);
  w[1] = tsp_pack_bf16(x[2], x[3]);
  w[2] = tsp_pack_bf16(x[4], x[5]);
  w[3] = tsp_pack_bf16(x[6], x[7]);
  return __builtin_bit_cast(tsp_bf16x8, w);
}

// ---- Delta_i = dO_i . O_i ------------------------------------------------------------
// One thread per 16 bytes of a (row, head) vector; the DH/8 threads of a vector are
// consecutive lanes of one wave and reduce with xor shuffles.
template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_delta_bf16_kernel(TspBwdParams p) {
  constexpr int TPR = DH / 8;
  static_assert(64 % TPR == 0, "a vector must not straddle two waves");
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = tid / TPR;  // (b * S_local + i) * Hq + h
  const int c = (int)(tid % TPR);
  const bool valid = row < p.n_rows;
  float acc = 0.f;
  if (valid) {
    const int64_t off = row * DH + c * 8;
    const tsp_u32x4 o = *reinterpret_cast<const tsp_u32x4*>(static_cast<const uint16_t*>(p.f.out) + off);
    const tsp_u32x4 d = *reinterpret_cast<const tsp_u32x4*>(static_cast<const uint16_t*>(p.dout) + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(o[w] << 16), __uint_as_float(d[w] << 16), acc);
      acc = fmaf(__uint_as_float(o[w] & 0xffff0000u), __uint_as_float(d[w] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (valid && c == 0) {
    const int32_t h = (int32_t)(row % p.f.Hq);
    const int64_t bi = row / p.f.Hq;
    const int32_t i = (int32_t)(bi % p.f.S_local);
    const int64_t b = bi / p.f.S_local;
    p.delta[(b * p.f.Hq + h) * p.f.S_local + i] = acc;
  }
}

// ---- dK / dV: key-stationary ---------------------------------------------------------
template <int DH, int NW>
struct BwdQTile {
  static constexpr int BQ = 32;                     // query rows per step
  static constexpr int ROW_BYTES = DH * 2;
  static constexpr int CPR = DH / 8;                // 16-byte chunks per row
  static constexpr int RPL = 64 / CPR;              // rows per 1 KiB wave-load
  static constexpr int TILE_BYTES = BQ * ROW_BYTES;
  static constexpr int WL = TILE_BYTES / 1024;      // wave-loads per tile
  static constexpr int LPW = 2 * WL / NW;           // Q + dO wave-loads per wave per stage
  static constexpr int META_BYTES = 256;            // per wave: 32 lse + 32 Delta
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES + NW * META_BYTES;
  static_assert((2 * WL) % NW == 0, "stage loads must split evenly over the waves");
};

// PIPE: issue the next step's S / dP products ahead of the current step's VALU work (one
// more score tile live; off where the registers do not allow it).
// MODE: which gradients one launch computes. Both (S, dP, P, dS, dV and dK) with K and V in
// registers need about 300 registers per lane at dh 128, one wave per SIMD; with V parked
// in LDS (VLDS) they fit in 256, two waves per SIMD, the form used at dh <= 128. dV alone
// (S, P, dV) and dK alone (S, dP, P, dS, dK) also fit in 256 with K and V in registers, as
// two launches that compute S twice.
enum BwdKvMode : int { BWD_KV_BOTH = 0, BWD_KV_DV = 1, BWD_KV_DK = 2 };

// VLDS (both gradients only): each lane parks its key's V row in LDS instead of registers
// (NKK x 16 bytes per lane, laid out lane-linear, read back by the same lane only), which
// brings the one-launch kernel down to the registers of two waves per SIMD.
template <int DH, int NW, int NBUF, bool PIPE, int MODE, int OCC, bool VLDS = false>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bwd_dkv_bf16_kernel(TspBwdParams bp) {
  using T = BwdQTile<DH, NW>;
  constexpr bool DO_DV = MODE != BWD_KV_DK, DO_DK = MODE != BWD_KV_DV;
  static_assert(!VLDS || MODE == BWD_KV_BOTH, "V in LDS is for the one-launch kernel");
  constexpr int VL_BYTES = VLDS ? NW * (DH / 16) * 1024 : 0;  // the parked V rows
  constexpr int NDB = DH / 32, NKK = DH / 16, PD = NBUF - 1, KB = 32 * NW;
  constexpr int VM_STAGE = T::LPW + 1;  // loads per wave per stage (tiles + metadata)
  // unroll the step loop over whole ring cycles (constant LDS slots) where the registers allow
  constexpr bool UNROLL_RING = DH <= 128 && (PIPE ? TSP_BWD_UNROLL_RING_PIPE : TSP_BWD_UNROLL_RING_NOPIPE);
  static_assert(PD >= 2 && VM_STAGE * (PD - 1) < 64, "ring depth / vmcnt range");
  const TspParams& p = bp.f;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * T::STAGE_BYTES + VL_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  // this lane's parked V row: 16 bytes per reduction step kk at vls + 1024 * kk
  uint8_t* const vls = smem + NBUF * T::STAGE_BYTES + wave * (DH / 16) * 1024 + lane * 16;

  int32_t unit = tsp_xcd_unit(blockIdx.x, gridDim.x);
  const int32_t kblk = unit % bp.n_kblocks;
  unit /= bp.n_kblocks;
  const int32_t hk = unit % p.Hkv;
  const int32_t b = unit / p.Hkv;
  const int32_t j0 = kblk * KB;                // first key of the workgroup
  const int32_t key = j0 + 32 * wave + col;   // this lane's key
  const int64_t kv_row = (int64_t)p.Hkv * DH;
  uint16_t* __restrict__ dkg = static_cast<uint16_t*>(bp.dk);
  uint16_t* __restrict__ dvg = static_cast<uint16_t*>(bp.dv);
  const int64_t o_off = ((int64_t)b * p.S_total + key) * kv_row + (int64_t)hk * DH + 4 * half;

  if (j0 >= bp.kv_need) {  // no local row sees these keys: zero partial gradients
    if (key < p.S_total) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if constexpr (DO_DK) *reinterpret_cast<tsp_u32x2*>(dkg + o_off + db * 32 + 8 * a) = tsp_u32x2{0u, 0u};
          if constexpr (DO_DV) *reinterpret_cast<tsp_u32x2*>(dvg + o_off + db * 32 + 8 * a) = tsp_u32x2{0u, 0u};
        }
    }
    return;
  }

  // K and V of this lane's key: B operands (k = dims 16kk + 8*half .. +8, column = key)
  tsp_bf16x8 kf[NKK], vf[NKK];
  {
    const int32_t keyc = min(key, p.S_total - 1);
    const int64_t off = ((int64_t)b * p.S_total + keyc) * kv_row + (int64_t)hk * DH + 8 * half;
    const uint16_t* kp = static_cast<const uint16_t*>(p.k) + off;
    const uint16_t* vp = static_cast<const uint16_t*>(p.v) + off;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[kk] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(kp + 16 * kk));
      if constexpr (VLDS) *reinterpret_cast<tsp_u32x4*>(vls + 1024 * kk) = *reinterpret_cast<const tsp_u32x4*>(vp + 16 * kk);
      else if constexpr (DO_DK) vf[kk] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(vp + 16 * kk));
    }
  }
  // Let these loads land here, once: otherwise the compiler waits for them (vmcnt) before
  // their first use inside the step loop, on every step, and that count also covers the
  // stage loads issued just before, so each step would wait for its own prefetch.
  tsp_wait_vm<0>();

  // Query tiles to sweep: local rows are increasing in position, so the rows that see
  // key j0 are a suffix; it starts in the first chunk if j0 lies below that chunk's end.
  const int32_t C = p.C;
  const int32_t first_row =
      j0 < (p.rank + 1) * C ? max(0, j0 - p.rank * C) : C + max(0, j0 - (2 * p.D - 1 - p.rank) * C);
  const int32_t t_first = first_row / 32;
  const int32_t n_qt = (p.S_local + 31) / 32;
  const int32_t tiles = n_qt - t_first;
  const int32_t n_steps = p.grp * tiles;  // step u: head hk*grp + u/tiles, tile t_first + u%tiles

  // ---- per-lane LDS offsets -------------------------------------------------------------
  // At dh 256 (its registers are short) one offset per 16-chunk swizzle period: the
  // swizzle only changes the low 4 bits of the chunk index, so chunks 16 apart lie 256
  // bytes apart and QP (TP) offsets serve all NKK (NDB) operands.
  constexpr int QP = DH == 256 ? NKK / 2 : NKK, TP = DH == 256 ? NDB / 2 : NDB;
  // RA: every LDS operand of the products read RAW products ahead of its product, in an
  // order held by scheduling barriers. The compiler's own order read each one just before its
  // product, so at one wave per SIMD (dh 256) every product waited the full LDS latency; at
  // two waves (the dh-128 one-launch kernel, V parked in LDS) the other wave hid only part
  // of it. Three products ahead is what the dh-128 kernel's registers allow without a spill
  // in its step loop.
  constexpr bool RA = (DH == 256 && !VLDS || DH == 128 && VLDS) && TSP_BWD_READ_AHEAD;
  constexpr int RAW = DH == 256 ? 4 : 3;
  int qoff[QP];  // row-wise A operand read: row `col`, chunk 2kk + half
#pragma unroll
  for (int kk = 0; kk < QP; ++kk)
    qoff[kk] = col * T::ROW_BYTES + (((2 * kk + half) ^ tsp_swz_rt<T::CPR>(col)) << 4);
  auto qo = [&](int kk) __attribute__((always_inline)) { return qoff[kk % QP] + (kk / QP) * 256; };
  int tlo[NDB], thi[NDB];  // transposing reads (the first TP are used)
  tsp_tr_offsets<DH>(lane, tlo, thi);

  // ---- this wave's share of a stage load --------------------------------------------------
  // Wave-load q of a stage is 1 KiB of the Q tile (q < QW) or the dO tile, rows
  // r0 + m * RSTEP with m = q mod QW and r0 the lane's row in the first one. Where a wave's
  // loads of a tile lie less than 16 rows apart (QW <= DP; the dh-128 one-launch kernel, one
  // load per tile) one lane offset per m serves both tiles: two registers fewer than an
  // offset and a row per load. Otherwise (dh 256: rows 16 apart share a swizzle, but moving
  // the row shift into the base ran 1.3% slower; dh 64: the waves do not divide a tile's
  // loads) each load keeps its own row and offset.
  const int64_t q_row_elems = (int64_t)p.Hq * DH;
  const uint32_t q_row_bytes = (uint32_t)(q_row_elems * 2);
  constexpr int QW = T::WL % NW == 0 ? T::WL / NW : 1, RSTEP = NW * T::RPL;
  constexpr int DP = RSTEP >= 16 ? 1 : 16 / RSTEP;
  constexpr bool SHARED = T::WL % NW == 0 && QW <= DP;
  const int r0 = wave * T::RPL + lane / T::CPR;
  uint32_t dma_lo[SHARED ? QW : 1];  // shared form: lane offset of the row r0 + m * RSTEP
  constexpr int LG = SHARED ? 1 : T::LPW;
  uint32_t dma_voff[LG];  // general form: row, lane offset, tile and slot of each load
  int dma_row[LG];
  bool dma_isdo[LG];
  uint32_t dma_slot[LG];
  if constexpr (SHARED) {
#pragma unroll
    for (int m = 0; m < QW; ++m) {
      const int row = r0 + m * RSTEP;
      dma_lo[m] = (uint32_t)row * q_row_bytes + (uint32_t)(((lane % T::CPR) ^ tsp_swz_rt<T::CPR>(row)) * 16);
    }
  } else {
#pragma unroll
    for (int q = 0; q < T::LPW; ++q) {
      const int i = q * NW + wave;
      const bool isdo = i >= T::WL;
      const int j = isdo ? i - T::WL : i;
      const int row = j * T::RPL + lane / T::CPR;
      const int c = (lane % T::CPR) ^ tsp_swz_rt<T::CPR>(row);
      dma_row[q] = row;
      dma_isdo[q] = isdo;
      dma_voff[q] = (uint32_t)row * q_row_bytes + (uint32_t)(c * 16);
      dma_slot[q] = (isdo ? T::TILE_BYTES : 0) + j * 1024;
    }
  }
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(tsp_lds_addr(smem));
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ dog = static_cast<const uint16_t*>(bp.dout);

  auto issue = [&](int u) __attribute__((always_inline)) {
    const uint32_t base = smem_addr + (u % NBUF) * T::STAGE_BYTES;  // the slot of stage u
    u = min(u, n_steps - 1);  // past the end: a duplicate of the last stage into that free slot
    const int32_t hl = u / tiles;
    const int32_t i0 = (t_first + u % tiles) * 32;
    const int32_t h = hk * p.grp + hl;
    const int64_t tbase = ((int64_t)b * p.S_local + i0) * q_row_elems + (int64_t)h * DH;
    if constexpr (!SHARED) {
#pragma unroll
      for (int q = 0; q < T::LPW; ++q) {
        const int32_t over = max(0, i0 + dma_row[q] - (p.S_local - 1));  // rows past the last
        tsp_lds_dma16((dma_isdo[q] ? dog : qg) + tbase, dma_voff[q] - (uint32_t)over * q_row_bytes,
                      base + dma_slot[q]);
      }
    } else {  // the lane offset carries the load's whole row; rows past the last read the last
#pragma unroll
      for (int q = 0; q < T::LPW; ++q) {
        const int m = q % QW;
        const bool isdo = q >= QW;
        const int32_t over = max(0, i0 + r0 + m * RSTEP - (p.S_local - 1));  // rows past the last
        tsp_lds_dma16((isdo ? dog : qg) + tbase, dma_lo[m] - (uint32_t)over * q_row_bytes,
                      base + (isdo ? T::TILE_BYTES : 0) + (m * NW + wave) * 1024);
      }
    }
    // lse (lanes 0..31) and Delta (lanes 32..63) of the tile's rows, into this wave's slot
    const int32_t ri = min(i0 + col, p.S_local - 1);
    const int64_t mi = ((int64_t)b * p.Hq + h) * p.S_local + ri;
    const float* src = half ? bp.delta + mi : p.lse + mi;
    tsp_lds_dma4(src, base + 2 * T::TILE_BYTES + wave * T::META_BYTES);
  };

  tsp_f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[db][e] = 0.f;
      dv[db][e] = 0.f;
    }

  const int32_t wave_key_max = j0 + 32 * wave + 31;

  // Every stage is addressed through its slot's base pointer: the loop below is unrolled
  // over the ring, so for most steps the slot is a constant folded into the LDS
  // instructions' offsets instead of an address add per read.
  auto slot = [&](int t) __attribute__((always_inline)) { return smem + (t % NBUF) * T::STAGE_BYTES; };

  // The wave's metadata of a stage holds lse (lanes 0..31) then Delta (lanes 32..63) of the
  // tile's rows; once the stage has landed the wave turns its lse values into
  // -lse * log2(e), the exponent offset of the weights (one multiply per stage instead of
  // one per weight).
  const float meta_scale = half ? 1.0f : -TSP_LOG2E;
  auto prescale_meta = [&](const uint8_t* qs) __attribute__((always_inline)) {
    // The lane's byte offset is formed here each time: a slot's metadata may lie past the
    // 16-bit LDS offset field, and an address kept live per slot across the loop was spilled
    // (its reload waits on vmcnt, which also drains the stage loads in flight).
    uint32_t l4 = 4u * (uint32_t)lane;
    asm volatile("" : "+v"(l4));
    float* m = reinterpret_cast<float*>(const_cast<uint8_t*>(qs) + 2 * T::TILE_BYTES + wave * T::META_BYTES + l4);
    *m = *m * meta_scale;
  };

  // S = Q K^T and dP = dO V^T of the stage at qs: lane holds key `col`, query rows
  // 8(e/4) + 4*half + e%4 of the step's tile
  auto sdp = [&](const uint8_t* qs, tsp_f32x16& s, tsp_f32x16& dp) __attribute__((always_inline)) {
    const uint8_t* ds = qs + T::TILE_BYTES;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      dp[e] = 0.f;
    }
    if constexpr (RA) {  // S then dP operands (and the parked V rows), each read RAW products ahead
      constexpr int NP = DO_DK ? 2 * NKK : NKK;
      tsp_bf16x8 ra[NP], rv[VLDS ? NP : 1];
      auto rd = [&](int j) __attribute__((always_inline)) {
        ra[j] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>((j < NKK ? qs : ds) + qo(j % NKK)));
        if constexpr (VLDS) {
          if (j >= NKK) rv[j] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(vls + 1024 * (j - NKK)));
        }
      };
#pragma unroll
      for (int j = 0; j < RAW; ++j) rd(j);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if (j + RAW < NP) rd(j + RAW);
        if (j < NKK) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[j], kf[j], s, 0, 0, 0);
        else if constexpr (VLDS) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[j], rv[j], dp, 0, 0, 0);
        else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[j], vf[j - NKK], dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const tsp_bf16x8 qa = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(qs + qo(kk)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s, 0, 0, 0);
    }
    if constexpr (DO_DK) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const tsp_bf16x8 da = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(ds + qo(kk)));
        const tsp_bf16x8 vb =
            VLDS ? __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(vls + 1024 * kk)) : vf[kk];
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb, dp, 0, 0, 0);
      }
    }
  };

  // P = exp2(s * log2(e)/sqrt(dh) - lse * log2(e)) on visible pairs, dS = P (dP - Delta),
  // then dV^T += dO^T P and dK^T += Q^T dS (rows = dims, columns = keys)
  auto grads = [&](int t, const uint8_t* qs, const tsp_f32x16& s, const tsp_f32x16& dp) __attribute__((always_inline)) {
    const uint8_t* ds = qs + T::TILE_BYTES;
    const float* meta = reinterpret_cast<const float*>(qs + 2 * T::TILE_BYTES + wave * T::META_BYTES);
    const int32_t i0 = (t_first + t % tiles) * 32;
    const int32_t pos0 = tsp_zigzag_position(i0, C, p.D, p.rank);
    const bool irregular = i0 + 31 >= p.S_local || (i0 < C && i0 + 31 >= C);
    // exponent arguments of the lane's 16 rows (the metadata holds -lse * log2(e))
    float x[16], del[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const tsp_f32x4 nl4 = *reinterpret_cast<const tsp_f32x4*>(meta + 8 * a + 4 * half);
      const tsp_f32x4 del4 = *reinterpret_cast<const tsp_f32x4*>(meta + 32 + 8 * a + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[4 * a + e] = fmaf(s[4 * a + e], p.scale_log2, nl4[e]);
        del[4 * a + e] = del4[e];
      }
    }
    // causal mask (steps that reach past a row's position, and irregular tiles that hold
    // a chunk boundary or rows past the last): masked arguments become -inf, weight 0. Both
    // cases are rare, wave-uniform branches; the empty asm keeps the compiler from turning
    // them into selects executed on every step.
    if (__builtin_expect(irregular, 0)) {
      asm volatile("");
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int32_t row = i0 + 8 * (v >> 2) + 4 * half + (v & 3);
        const int32_t pos = tsp_zigzag_position(min(row, p.S_local - 1), C, p.D, p.rank);
        if (row >= p.S_local || key > pos) x[v] = -INFINITY;
      }
    } else if (__builtin_expect(wave_key_max > pos0, 0)) {
      asm volatile("");
      const int32_t lim = key - pos0 - 4 * half;  // row offsets below this see no key
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) < lim) x[v] = -INFINITY;
    }
    // RA: the transposed operands of the dV / dK products (dV then dK for each (st, db), the
    // order below), the first RAW read ahead of the weights and each later one RAW products
    // ahead of its product
    constexpr int NT = (DO_DV ? 1 : 0) + (DO_DK ? 1 : 0), NPT = 2 * NDB * NT;
    tsp_bf16x8 tb[RA ? NPT : 1];
    auto trd = [&](int j) __attribute__((always_inline)) {
      const int st = (j / NT) / NDB, db = (j / NT) % NDB;
      const bool is_dv = DO_DV && (NT == 1 || j % 2 == 0);
      const int ro = st * 16 * T::ROW_BYTES + (db / TP) * 256;
      const uint8_t* base = is_dv ? ds : qs;
      return tsp_tr_read8(base + tlo[db % TP] + ro, base + thi[db % TP] + ro);
    };
    if constexpr (RA) {
#pragma unroll
      for (int j = 0; j < RAW; ++j) tb[j] = trd(j);
    }
    float pw[16], dsw[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pw[v] = tsp_exp2(x[v]);
      if constexpr (DO_DK) dsw[v] = pw[v] * (dp[v] - del[v]);
    }
    tsp_bf16x8 pf[2], dsf[2];
    if constexpr (DO_DV) {
      pf[0] = tsp_pack8(pw);
      pf[1] = tsp_pack8(pw + 8);
    }
    if constexpr (DO_DK) {
      dsf[0] = tsp_pack8(dsw);
      dsf[1] = tsp_pack8(dsw + 8);
    }
    if constexpr (RA) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        if (j + RAW < NPT) tb[j + RAW] = trd(j + RAW);
        const int st = (j / NT) / NDB, db = (j / NT) % NDB;
        if (DO_DV && (NT == 1 || j % 2 == 0)) dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[j], pf[st], dv[db], 0, 0, 0);
        else dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[j], dsf[st], dk[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int ro = st * 16 * T::ROW_BYTES + (db / TP) * 256;
        if constexpr (DO_DV) {
          const tsp_bf16x8 doT = tsp_tr_read8(ds + tlo[db % TP] + ro, ds + thi[db % TP] + ro);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(doT, pf[st], dv[db], 0, 0, 0);
        }
        if constexpr (DO_DK) {
          const tsp_bf16x8 qT = tsp_tr_read8(qs + tlo[db % TP] + ro, qs + thi[db % TP] + ro);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, dsf[st], dk[db], 0, 0, 0);
        }
      }
  };

  // Step t (PIPE): the S / dP products of step t+1 go to the matrix pipe ahead of step t's
  // VALU work, then step t's dV / dK products. Stages t and t+1 are read in step t, so the
  // stage issued here, NBUF-1 ahead, takes the slot of stage t-1.
  auto step = [&](int t, const uint8_t* cur, const uint8_t* nxt, tsp_f32x16& sc, tsp_f32x16& dc, tsp_f32x16& sn,
                  tsp_f32x16& dn) __attribute__((always_inline)) {
    tsp_wait_vm<VM_STAGE * (PD - 2)>();  // stage t+1 landed (this wave's part)
    __syncthreads();                     // ... for every wave; every wave is past step t-1
    prescale_meta(nxt);
    issue(t + PD);
    sdp(nxt, sn, dn);  // past the last step this reads a duplicate stage; unused
    grads(t, cur, sc, dc);
  };
  // Step t without the pipeline: one stage per step.
  auto step1 = [&](int t, const uint8_t* cur) __attribute__((always_inline)) {
    tsp_wait_vm<VM_STAGE * (PD - 1)>();  // stage t landed (this wave's part)
    __syncthreads();                     // ... for every wave; the slot of stage t-1 is free
    prescale_meta(cur);
    issue(t + PD);
    tsp_f32x16 s0, d0;
    sdp(cur, s0, d0);
    grads(t, cur, s0, d0);
  };

#pragma unroll 1
  for (int u = 0; u < PD; ++u) issue(u);
  static_assert(!PIPE || NBUF % 2 == 0, "the unrolled groups keep the two score tiles' roles");
  if constexpr (PIPE) {
    tsp_wait_vm<VM_STAGE * (PD - 1)>();
    __syncthreads();
    prescale_meta(smem);
    tsp_f32x16 s0, d0, s1, d1;
    sdp(smem, s0, d0);
    int t = 0;
    // whole ring cycles: the slots are compile-time constants
#pragma unroll 1
    for (; UNROLL_RING && t + NBUF <= n_steps; t += NBUF)
      [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
        ((Us % 2 == 0 ? step(t + Us, smem + Us * T::STAGE_BYTES, smem + ((Us + 1) % NBUF) * T::STAGE_BYTES, s0, d0, s1, d1)
                      : step(t + Us, smem + Us * T::STAGE_BYTES, smem + ((Us + 1) % NBUF) * T::STAGE_BYTES, s1, d1, s0, d0)),
         ...);
      }(std::make_integer_sequence<int, NBUF>{});
#pragma unroll 1
    for (; t + 2 <= n_steps; t += 2) {
      step(t, slot(t), slot(t + 1), s0, d0, s1, d1);
      step(t + 1, slot(t + 1), slot(t + 2), s1, d1, s0, d0);
    }
    if (t < n_steps) step(t, slot(t), slot(t + 1), s0, d0, s1, d1);
  } else {
    int t = 0;
#pragma unroll 1
    for (; UNROLL_RING && t + NBUF <= n_steps; t += NBUF)
      [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
        (step1(t + Us, smem + Us * T::STAGE_BYTES), ...);
      }(std::make_integer_sequence<int, NBUF>{});
#pragma unroll 1
    for (; t < n_steps; ++t) step1(t, slot(t));
  }
  tsp_wait_vm<0>();  // the trailing duplicate loads land before the workgroup ends

  if (key < p.S_total) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        tsp_u32x2 wk, wv;
        wk[0] = tsp_pack_bf16(dk[db][4 * a] * bp.scale, dk[db][4 * a + 1] * bp.scale);
        wk[1] = tsp_pack_bf16(dk[db][4 * a + 2] * bp.scale, dk[db][4 * a + 3] * bp.scale);
        wv[0] = tsp_pack_bf16(dv[db][4 * a], dv[db][4 * a + 1]);
        wv[1] = tsp_pack_bf16(dv[db][4 * a + 2], dv[db][4 * a + 3]);
        if constexpr (DO_DK) *reinterpret_cast<tsp_u32x2*>(dkg + o_off + db * 32 + 8 * a) = wk;
        if constexpr (DO_DV) *reinterpret_cast<tsp_u32x2*>(dvg + o_off + db * 32 + 8 * a) = wv;
      }
  }
}

// ---- dQ: query-stationary ------------------------------------------------------------
template <int DH, int NW>
struct BwdKvTile {
  static constexpr int BK = 32;                     // keys per step and stage
  static constexpr int ROW_BYTES = DH * 2;
  static constexpr int CPR = DH / 8;
  static constexpr int RPL = 64 / CPR;
  static constexpr int TILE_BYTES = BK * ROW_BYTES;
  static constexpr int WL = TILE_BYTES / 1024;
  static constexpr int LPW = 2 * WL / NW;           // K + V wave-loads per wave per stage
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int SWZ = CPR < 16 ? CPR : 16;
  static_assert((2 * WL) % NW == 0, "stage loads must split evenly over the waves");
  // V is only read row-wise: 16 consecutive rows at one chunk hit 16 distinct chunks
  __device__ static int swz_v(int row) { return row & (SWZ - 1); }
};

template <int DH, int NW, int NBUF, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bwd_dq_bf16_kernel(TspBwdParams bp) {
  using T = BwdKvTile<DH, NW>;
  constexpr int NDB = DH / 32, NKK = DH / 16, PD = NBUF - 1, BK = T::BK;
  constexpr int VM_STAGE = T::LPW;
  static_assert(VM_STAGE * (PD - 1) < 64, "vmcnt range");
  // RA (one wave per SIMD): every LDS operand read RAW products ahead of its product, held
  // by scheduling barriers (the compiler's order waited the full LDS latency per product)
  constexpr bool RA = OCC == 1 && TSP_BWD_READ_AHEAD;
  constexpr int RAW = 4;
  const TspParams& p = bp.f;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * T::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  int32_t unit = tsp_xcd_unit(blockIdx.x, gridDim.x);
  const int32_t pair = unit % p.n_pairs;
  unit /= p.n_pairs;
  const int32_t hgrp = unit % p.n_hgroups;
  unit /= p.n_hgroups;
  const int32_t hk = unit % p.Hkv;
  const int32_t b = unit / p.Hkv;

  const int64_t kv_row = (int64_t)p.Hkv * DH;
  const uint32_t kv_row_bytes = (uint32_t)(kv_row * 2);
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.S_total * p.Hkv + hk) * DH;
  const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.S_total * p.Hkv + hk) * DH;
  const int pos_blocks = p.BQ / 32;

  int koff[NKK], voff[NKK];  // row-wise A operand reads of K and V: row `col`, chunk 2kk + half
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    koff[kk] = col * T::ROW_BYTES + (((2 * kk + half) ^ tsp_swz_rt<T::CPR>(col)) << 4);
    voff[kk] = T::TILE_BYTES + col * T::ROW_BYTES + (((2 * kk + half) ^ T::swz_v(col)) << 4);
  }
  int tlo[NDB], thi[NDB];  // transposing reads of K
  tsp_tr_offsets<DH>(lane, tlo, thi);

  uint32_t dma_voff[T::LPW];
  int dma_row[T::LPW];
  bool dma_isv[T::LPW];
  uint32_t dma_slot[T::LPW];
#pragma unroll
  for (int q = 0; q < T::LPW; ++q) {
    const int i = q * NW + wave;
    const bool isv = i >= T::WL;
    const int j = isv ? i - T::WL : i;
    const int row = j * T::RPL + lane / T::CPR;
    const int c = (lane % T::CPR) ^ (isv ? T::swz_v(row) : tsp_swz_rt<T::CPR>(row));
    dma_row[q] = row;
    dma_isv[q] = isv;
    dma_voff[q] = (uint32_t)row * kv_row_bytes + (uint32_t)(c * 16);
    dma_slot[q] = (isv ? T::TILE_BYTES : 0) + j * 1024;
  }
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(tsp_lds_addr(smem));

  for (int which = 0; which < 2; ++which) {
    const int32_t qt = which == 0 ? p.n_qtiles - 1 - pair : pair;
    if (which == 1 && qt == p.n_qtiles - 1 - pair) break;  // middle tile of an odd count
    const int32_t row0 = qt * p.BQ;
    const int32_t last_row = min(row0 + p.BQ, p.S_local) - 1;
    const int32_t kv_end = tsp_zigzag_position(last_row, p.C, p.D, p.rank) + 1;
    const int32_t n_steps = (kv_end + BK - 1) / BK;

    const int pb = wave % pos_blocks, hh = wave / pos_blocks;
    const int32_t head = hk * p.grp + hgrp * p.GH + hh;
    const int32_t first = row0 + pb * 32;
    const int32_t r = first + col;
    const bool rvalid = r < p.S_local;
    const int32_t lrow = min(r, p.S_local - 1);
    const int32_t qpos = tsp_zigzag_position(lrow, p.C, p.D, p.rank);
    const bool wave_active = first < p.S_local;
    const int32_t wave_min_pos = tsp_zigzag_position(min(first, p.S_local - 1), p.C, p.D, p.rank);
    const int32_t wave_max_pos = tsp_zigzag_position(min(first + 31, p.S_local - 1), p.C, p.D, p.rank);
    const int32_t t_mask = max(0, wave_min_pos + 1) / BK;  // steps before it need no mask

    // Q^T and dO^T operands (column = query `col`, k = dims 16kk + 8*half .. +8)
    tsp_bf16x8 qf[NKK], dof[NKK];
    const int64_t qo = (((int64_t)b * p.S_local + lrow) * p.Hq + head) * DH + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = __builtin_bit_cast(tsp_bf16x8,
                                  *reinterpret_cast<const tsp_u32x4*>(static_cast<const uint16_t*>(p.q) + qo + 16 * kk));
      dof[kk] = __builtin_bit_cast(
          tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(static_cast<const uint16_t*>(bp.dout) + qo + 16 * kk));
    }
    const int64_t li = ((int64_t)b * p.Hq + head) * p.S_local + lrow;
    const float lse2 = p.lse[li] * TSP_LOG2E;
    const float delta = bp.delta[li];
    tsp_wait_vm<0>();  // these loads land here, not behind a wait in every step (see the dK/dV kernel)

    tsp_f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

    auto issue = [&](int s) {
      const uint32_t base = smem_addr + (s % NBUF) * T::STAGE_BYTES;  // the slot of stage s
      s = min(s, n_steps - 1);  // past the end: a duplicate of the last stage into that free slot
      const int32_t kv0 = s * BK;
#pragma unroll
      for (int q = 0; q < T::LPW; ++q) {
        const int32_t over = max(0, kv0 + dma_row[q] - (kv_end - 1));  // rows past the last key
        tsp_lds_dma16((dma_isv[q] ? vbase : kbase) + (int64_t)kv0 * kv_row,
                      dma_voff[q] - (uint32_t)over * kv_row_bytes, base + dma_slot[q]);
      }
    };

    // Step t: wait for its stage, barrier, load the stage PD ahead, then S^T = K Q^T and
    // dP^T = V dO^T (lane holds query `col`, keys 8(e/4) + 4*half + e%4), dS^T, and
    // dQ^T += K^T dS^T (rows = dims, columns = queries). MASK: the step reaches past some
    // row's position; the unmasked steps come first and run in their own loop, so they
    // carry no compare or select. Waves whose rows see none of a step's keys only take
    // part in its barrier.
    auto run = [&](int t, auto mask_const) {
      constexpr bool MASK = decltype(mask_const)::value;
      tsp_wait_vm<VM_STAGE * (PD - 1)>();
      __syncthreads();
      issue(t + PD);
      if (!wave_active || t * BK > wave_max_pos) return;

      const uint8_t* st8 = smem + (t % NBUF) * T::STAGE_BYTES;
      tsp_f32x16 sT, dpT;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sT[e] = 0.f;
        dpT[e] = 0.f;
      }
      // the transposed K operands of the dQ products: with RA the first RAW are read ahead of
      // the weights
      tsp_bf16x8 tb[RA ? 2 * NDB : 1];
      auto trd = [&](int j) __attribute__((always_inline)) {  // product j: (st, db) = (j / NDB, j % NDB)
        const int ro = (j / NDB) * 16 * T::ROW_BYTES;
        return tsp_tr_read8(st8 + tlo[j % NDB] + ro, st8 + thi[j % NDB] + ro);
      };
      if constexpr (RA) {  // S^T then dP^T operands, each read RAW products ahead
        tsp_bf16x8 ra[2 * NKK];
        auto rd = [&](int j) __attribute__((always_inline)) {
          return __builtin_bit_cast(tsp_bf16x8,
                                    *reinterpret_cast<const tsp_u32x4*>(st8 + (j < NKK ? koff[j] : voff[j - NKK])));
        };
#pragma unroll
        for (int j = 0; j < RAW; ++j) ra[j] = rd(j);
#pragma unroll
        for (int j = 0; j < 2 * NKK; ++j) {
          if (j + RAW < 2 * NKK) ra[j + RAW] = rd(j + RAW);
          if (j < NKK) sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[j], qf[j], sT, 0, 0, 0);
          else dpT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[j], dof[j - NKK], dpT, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < RAW; ++j) tb[j] = trd(j);
      } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const tsp_bf16x8 ka = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st8 + koff[kk]));
          sT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], sT, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const tsp_bf16x8 va = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st8 + voff[kk]));
          dpT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[kk], dpT, 0, 0, 0);
        }
      }
      float dsw[16];
      const int32_t hi = qpos - t * BK - 4 * half;  // key offset limit of this lane
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float pv = tsp_exp2(fmaf(sT[e], p.scale_log2, -lse2));
        if constexpr (MASK) {
          if (8 * (e >> 2) + (e & 3) > hi) pv = 0.f;
        }
        dsw[e] = pv * (dpT[e] - delta);
      }
      tsp_bf16x8 dsf[2];
      dsf[0] = tsp_pack8(dsw);
      dsf[1] = tsp_pack8(dsw + 8);
      if constexpr (RA) {
#pragma unroll
        for (int j = 0; j < 2 * NDB; ++j) {
          if (j + RAW < 2 * NDB) tb[j + RAW] = trd(j + RAW);
          acc[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[j], dsf[j / NDB], acc[j % NDB], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int ro = st * 16 * T::ROW_BYTES;
          const tsp_bf16x8 kT = tsp_tr_read8(st8 + tlo[db] + ro, st8 + thi[db] + ro);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsf[st], acc[db], 0, 0, 0);
        }
    };

    __syncthreads();  // the previous tile's readers are done with every slot
#pragma unroll 1
    for (int s = 0; s < PD; ++s) issue(s);
    const int t_split = min(t_mask, n_steps);
    int t = 0;
#pragma unroll 1
    for (; t < t_split; ++t) run(t, std::false_type{});
#pragma unroll 1
    for (; t < n_steps; ++t) run(t, std::true_type{});
    tsp_wait_vm<0>();  // trailing duplicate loads land before the slots are reused

    if (wave_active && rvalid) {
      uint16_t* op = static_cast<uint16_t*>(bp.dq) + (((int64_t)b * p.S_local + lrow) * p.Hq + head) * DH + 4 * half;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          tsp_u32x2 w;
          w[0] = tsp_pack_bf16(acc[db][4 * a] * bp.scale, acc[db][4 * a + 1] * bp.scale);
          w[1] = tsp_pack_bf16(acc[db][4 * a + 2] * bp.scale, acc[db][4 * a + 3] * bp.scale);
          *reinterpret_cast<tsp_u32x2*>(op + db * 32 + 8 * a) = w;
        }
    }
  }
}

}  // namespace tsp
