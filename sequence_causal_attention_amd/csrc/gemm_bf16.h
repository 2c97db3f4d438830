// gemm_bf16.h -- C = A B^T for bf16 A [M, K] and B [N, K] (both K-contiguous, the layout of
// a token-major activation and of a [out_features, in_features] weight), fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Used by the per-rank attention layer of TSP ("Folding Tensor and Sequence Parallelism
// ...", section 2, attention layers: every rank projects its own sequence shard with each
// packed W_Q / W_K / W_V / W_O shard in turn): the Q / K / V projections of the rank's
// tokens and the output projection accumulated over the weight shards.
//
// Design: a workgroup computes a BM x BN tile of C with WM x WN waves, each a
// (BM / WM) x (BN / WN) block of 32 x 32 MFMA tiles. K advances in stages of 64 through a
// two-slot ring of LDS stages filled straight from global memory (global_load_lds_dwordx4,
// every wave an equal share; a wave waits for its own loads, then the barrier makes the
// stage whole). Rows are 128 bytes in LDS, chunk c of row r stored at c ^ ((r / 2) % 8), so
// 16 consecutive rows read at one logical chunk hit 16 distinct bank groups. Each wave
// computes D^T = B A^T per block, so a lane holds one row m of C and 4 consecutive columns
// n per register quad: 8-byte (bf16) or 16-byte (fp32) stores. Rows past M (or columns past
// N) are loaded clamped and never stored; K must be a multiple of 64.
//
// The big tile (256 x 256, 8 waves of 128 x 64) reads 6 KiB of LDS per wave per 16-deep
// k step for 8 MFMAs; the small one (128 x 128, 4 waves of 64 x 64) 4 KiB for 4 and serves
// launches with too few big tiles to cover the CUs.
//
// Column segments: the columns of C may be split into up to 3 consecutive segments, each
// with its own first row of B (B row of column n = b_row + n - segment start; segments in
// increasing B row order), its own destination (pointer, row stride) and row map (identity,
// or the zigzag map: row m = b * S_local + i goes to row b * S_total + g(i) of a
// [B, S_total, ...] buffer). One launch so computes a weight shard's Q (into a local
// buffer) and K, V (at the tokens' global positions in the gathered K / V buffers).
//
// Epilogue modes: store bf16; store fp32; add into fp32; add into fp32 and store the sum as
// bf16 into a second buffer (one segment only).
#pragma once

#include "attn_common.h"
#include "attn_fwd_bf16.h"

namespace tsp {

enum GemmMode : int32_t { GEMM_STORE_BF16 = 0, GEMM_STORE_F32 = 1, GEMM_ADD_F32 = 2, GEMM_ADD_F32_TO_BF16 = 3 };

constexpr int GEMM_MAX_SEG = 3;

struct GemmSeg {
  void* c;         // destination of the segment's column 0 (row 0), mode-dependent type
  int64_t ldc;     // its row stride (elements)
  int32_t n_end;   // one past the segment's last column of C
  int32_t b_row;   // row of B feeding the segment's column 0
  int32_t zigzag;  // 1: map output rows through the zigzag positions
  int32_t pad_;
};

struct GemmParams {
  const uint16_t* a;  // [M, K], row stride lda (elements)
  const uint16_t* b;  // B rows, row stride ldb
  void* c2;           // GEMM_ADD_F32_TO_BF16: the bf16 destination (segment 0's row stride)
  int64_t lda, ldb;
  int32_t M, N, K;
  int32_t mode;
  int32_t nseg;
  int32_t S_total, C, D, rank, S_local;  // zigzag row map
  int32_t n_tiles_m, n_tiles_n;
  GemmSeg seg[GEMM_MAX_SEG];
};

constexpr int GEMM_BK = 64;

__device__ __forceinline__ int gemm_swz(int row) { return (row >> 1) & 7; }

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // a wave's block of C
  static constexpr int MB = TM / 32, NB = TN / 32;  // its 32 x 32 MFMA tiles
  static constexpr int A_BYTES = BM * GEMM_BK * 2;
  static constexpr int STAGE_BYTES = (BM + BN) * GEMM_BK * 2;
  static constexpr int NLOADS = (BM + BN) / 8;  // 1-KiB wave-loads (8 rows) per stage
  static constexpr int LPW = NLOADS / NW;
  static_assert(NLOADS % NW == 0, "stage loads must split evenly over the waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave blocks are whole MFMA tiles");
};

// Segment of column n (n < N): the first segment whose end lies above n.
__device__ __forceinline__ int gemm_seg_of(const GemmParams& p, int32_t n) {
  return (p.nseg > 1 && n >= p.seg[0].n_end) ? ((p.nseg > 2 && n >= p.seg[1].n_end) ? 2 : 1) : 0;
}

__device__ __forceinline__ int32_t gemm_b_row(const GemmParams& p, int32_t n) {
  const int s = gemm_seg_of(p, n);
  const int32_t start = s == 0 ? 0 : p.seg[s - 1].n_end;
  return p.seg[s].b_row + (n - start);
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_nt_bf16_kernel(GemmParams p) {
  using G = GemmCfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * G::STAGE_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;  // this wave's block

  // tiles: consecutive units stay on one XCD (shared L2); a run of units walks down a
  // column of up to 8 row tiles before moving right, so the XCD's units share B panels
  // and a few A panels
  const int32_t unit = tsp_xcd_unit(blockIdx.x, gridDim.x);
  constexpr int32_t GM = 8;
  const int32_t band = unit / (GM * p.n_tiles_n), in_band = unit % (GM * p.n_tiles_n);
  const int32_t band_rows = min(GM, p.n_tiles_m - band * GM);
  const int32_t tile_m = band * GM + in_band % band_rows, tile_n = in_band / band_rows;
  const int32_t m0 = tile_m * BM, n0 = tile_n * BN;

  // this wave's share of a stage: load i = q * NW + wave; loads below BM/8 fill the A tile
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(tsp_lds_addr(smem));
  const int32_t b_row0 = gemm_b_row(p, n0);  // segments ascend: the tile's lowest B row
  uint32_t dma_voff[G::LPW], dma_slot[G::LPW];
  bool dma_isb[G::LPW];
#pragma unroll
  for (int q = 0; q < G::LPW; ++q) {
    const int i = q * G::NW + wave;
    const bool isb = i >= BM / 8;
    const int j = isb ? i - BM / 8 : i;
    const int row = j * 8 + lane / 8;  // 8 rows of 128 bytes per 1 KiB load
    const int c = (lane % 8) ^ gemm_swz(row);
    // rows past M / N read the last row instead (never stored); offsets relative to the tile
    const uint32_t trow = isb ? (uint32_t)(gemm_b_row(p, min(n0 + row, p.N - 1)) - b_row0)
                              : (uint32_t)(min(m0 + row, p.M - 1) - m0);
    dma_isb[q] = isb;
    dma_voff[q] = trow * (uint32_t)((isb ? p.ldb : p.lda) * 2) + c * 16;
    dma_slot[q] = (isb ? G::A_BYTES : 0) + j * 1024;
  }
  const uint16_t* a_tile = p.a + (int64_t)m0 * p.lda;
  const uint16_t* b_tile = p.b + (int64_t)b_row0 * p.ldb;
  const int n_stages = p.K / GEMM_BK;
  auto issue = [&](int s) {
    const uint32_t base = smem_addr + (s & 1) * G::STAGE_BYTES;
    const int64_t k0 = (int64_t)min(s, n_stages - 1) * GEMM_BK;  // past the end: a duplicate
#pragma unroll
    for (int q = 0; q < G::LPW; ++q)
      tsp_lds_dma16((dma_isb[q] ? b_tile : a_tile) + k0, dma_voff[q], base + dma_slot[q]);
  };

  // operand reads: block rows (32 of them) `col`, logical chunk 2kk + half of the 16-k step
  int aoff[G::MB], boff[G::NB], rsw_a[G::MB], rsw_b[G::NB];
#pragma unroll
  for (int bi = 0; bi < G::MB; ++bi) {
    const int r = G::TM * wm + 32 * bi + col;
    aoff[bi] = r * 128;
    rsw_a[bi] = gemm_swz(r);
  }
#pragma unroll
  for (int bi = 0; bi < G::NB; ++bi) {
    const int r = G::TN * wn + 32 * bi + col;
    boff[bi] = G::A_BYTES + r * 128;
    rsw_b[bi] = gemm_swz(r);
  }

  tsp_f32x16 acc[G::NB][G::MB];
#pragma unroll
  for (int x = 0; x < G::NB; ++x)
#pragma unroll
    for (int y = 0; y < G::MB; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

  issue(0);
#pragma unroll 1
  for (int s = 0; s < n_stages; ++s) {
    tsp_wait_vm<0>();  // stage s landed (this wave's part)
    __syncthreads();   // ... for every wave; every wave is done with stage s-1
    issue(s + 1);      // into the other slot (past the end: a duplicate, drained below)
    const uint8_t* st = smem + (s & 1) * G::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < GEMM_BK / 16; ++kk) {
      tsp_bf16x8 av[G::MB], bv[G::NB];
#pragma unroll
      for (int bi = 0; bi < G::MB; ++bi)
        av[bi] = __builtin_bit_cast(
            tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st + aoff[bi] + (((2 * kk + half) ^ rsw_a[bi]) << 4)));
#pragma unroll
      for (int bi = 0; bi < G::NB; ++bi)
        bv[bi] = __builtin_bit_cast(
            tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st + boff[bi] + (((2 * kk + half) ^ rsw_b[bi]) << 4)));
#pragma unroll
      for (int x = 0; x < G::NB; ++x)
#pragma unroll
        for (int y = 0; y < G::MB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[x], av[y], acc[x][y], 0, 0, 0);
    }
  }
  tsp_wait_vm<0>();

  // epilogue: lane holds row m = m0 + TM wm + 32y + col, columns n0 + TN wn + 32x + 8a + 4half + 0..3
#pragma unroll
  for (int y = 0; y < G::MB; ++y) {
    const int32_t m = m0 + G::TM * wm + 32 * y + col;
    if (m >= p.M) continue;
    int64_t zrow = m;
    if (p.S_local > 0) {
      const int32_t bb = m / p.S_local, i = m - bb * p.S_local;
      zrow = (int64_t)bb * p.S_total + tsp_zigzag_position(i, p.C, p.D, p.rank);
    }
#pragma unroll
    for (int x = 0; x < G::NB; ++x)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int32_t n = n0 + G::TN * wn + 32 * x + 8 * a + 4 * half;
        if (n >= p.N) continue;  // segment ends are multiples of 4: a quad is in one segment
        const int s = gemm_seg_of(p, n);
        const int32_t cn = n - (s == 0 ? 0 : p.seg[s - 1].n_end);
        const int64_t off = (p.seg[s].zigzag ? zrow : (int64_t)m) * p.seg[s].ldc + cn;
        const float v0 = acc[x][y][4 * a], v1 = acc[x][y][4 * a + 1], v2 = acc[x][y][4 * a + 2],
                    v3 = acc[x][y][4 * a + 3];
        if (p.mode == GEMM_STORE_BF16) {
          *reinterpret_cast<tsp_u32x2*>(static_cast<uint16_t*>(p.seg[s].c) + off) =
              tsp_u32x2{tsp_pack_bf16(v0, v1), tsp_pack_bf16(v2, v3)};
        } else {
          float4* cp = reinterpret_cast<float4*>(static_cast<float*>(p.seg[s].c) + off);
          float4 r = make_float4(v0, v1, v2, v3);
          if (p.mode != GEMM_STORE_F32) {
            const float4 o = *cp;
            r = make_float4(o.x + v0, o.y + v1, o.z + v2, o.w + v3);
          }
          if (p.mode == GEMM_ADD_F32_TO_BF16)
            *reinterpret_cast<tsp_u32x2*>(static_cast<uint16_t*>(p.c2) + off) =
                tsp_u32x2{tsp_pack_bf16(r.x, r.y), tsp_pack_bf16(r.z, r.w)};
          else
            *cp = r;
        }
      }
  }
}

}  // namespace tsp
