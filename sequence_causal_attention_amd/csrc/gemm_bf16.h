// gemm_bf16.h -- C = A B^T for bf16 A [M, K] and B [N, K] (both K-contiguous, the layout of
// a token-major activation and of a [out_features, in_features] weight), fp32
// accumulation, on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Used by the per-rank attention layer of TSP ("Folding Tensor and Sequence Parallelism
// ...", section 2, attention layers: every rank projects its own sequence shard with each
// packed W_Q / W_K / W_V / W_O shard in turn): the Q / K / V projections of the rank's
// tokens and the output projection accumulated over the weight shards.
//
// Design: a workgroup computes a 128 x 128 tile of C with 4 waves of 64 x 64 (2 x 2 MFMA
// blocks). K advances in stages of 64 through a ring of LDS slots filled straight from
// global memory (global_load_lds_dwordx4, every wave an equal share, wait for exactly the
// stage needed next). Rows are 128 bytes in LDS, chunk c of row r stored at
// c ^ ((r / 2) % 8), so 16 consecutive rows read at one logical chunk hit 16 distinct bank
// groups. Each wave computes D^T = B A^T per block, so a lane holds one row m of C and 4
// consecutive columns n per register quad: 8-byte (bf16) or 16-byte (fp32) stores.
// Rows past M (or columns past N) are loaded clamped and never stored; K must be a
// multiple of 64 and lda, ldb at most 2^24 (per-lane 32-bit offsets within a tile).
//
// Epilogue modes: store bf16; store fp32; add into fp32; add into fp32 and store the sum as
// bf16 into a second buffer. An optional row map writes row m of C to row
// b * S_total + g(i) (m = b * 2C + i, g the zigzag map) of a [B, S_total, ...] buffer: the
// K / V projections of the rank's tokens land at their global positions in the gathered
// K / V buffer directly.
#pragma once

#include "attn_common.h"
#include "attn_fwd_bf16.h"

namespace tsp {

enum GemmMode : int32_t { GEMM_STORE_BF16 = 0, GEMM_STORE_F32 = 1, GEMM_ADD_F32 = 2, GEMM_ADD_F32_TO_BF16 = 3 };

struct GemmParams {
  const uint16_t* a;  // [M, K], row stride lda (elements)
  const uint16_t* b;  // [N, K], row stride ldb
  void* c;            // output rows (mode-dependent type), row stride ldc, column offset c_col
  void* c2;           // GEMM_ADD_F32_TO_BF16: the bf16 destination (same ldc / row map)
  int64_t lda, ldb, ldc, c_col;
  int32_t M, N, K;
  int32_t mode;
  int32_t zigzag;                      // 1: map output rows through the zigzag positions
  int32_t S_total, C, D, rank, S_local;  // row map: m = b * S_local + i -> b * S_total + g(i)
  int32_t n_tiles_n;                   // ceil(N / 128)
};

constexpr int GEMM_BM = 128, GEMM_BN = 128, GEMM_BK = 64, GEMM_NBUF = 2;
constexpr int GEMM_TILE_BYTES = GEMM_BM * GEMM_BK * 2;      // 16 KiB per operand tile
constexpr int GEMM_STAGE_BYTES = 2 * GEMM_TILE_BYTES;       // A tile then B tile
constexpr int GEMM_LPW = 2 * GEMM_TILE_BYTES / 1024 / 4;    // wave-loads per wave per stage

__device__ __forceinline__ int gemm_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(256, 2) void gemm_nt_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[GEMM_NBUF * GEMM_STAGE_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 64 x 64 quadrant

  const int32_t tile_m = blockIdx.x / p.n_tiles_n, tile_n = blockIdx.x % p.n_tiles_n;
  const int32_t m0 = tile_m * GEMM_BM, n0 = tile_n * GEMM_BN;

  // this wave's share of a stage: load i = q*4 + wave; loads 0..15 the A tile, 16..31 B
  const uint32_t smem_addr = __builtin_amdgcn_readfirstlane(tsp_lds_addr(smem));
  uint32_t dma_voff[GEMM_LPW], dma_slot[GEMM_LPW];
  bool dma_isb[GEMM_LPW];
#pragma unroll
  for (int q = 0; q < GEMM_LPW; ++q) {
    const int i = q * 4 + wave;
    const bool isb = i >= 16;
    const int j = isb ? i - 16 : i;
    const int row = j * 8 + lane / 8;  // 8 rows of 128 bytes per 1 KiB load
    const int c = (lane % 8) ^ gemm_swz(row);
    // rows past M / N read the last row instead (never stored); offsets relative to the tile
    const int trow = isb ? min(n0 + row, p.N - 1) - n0 : min(m0 + row, p.M - 1) - m0;
    dma_isb[q] = isb;
    dma_voff[q] = (uint32_t)(trow * (isb ? p.ldb : p.lda) * 2 + c * 16);
    dma_slot[q] = (isb ? GEMM_TILE_BYTES : 0) + j * 1024;
  }
  const uint16_t* a_tile = p.a + (int64_t)m0 * p.lda;
  const uint16_t* b_tile = p.b + (int64_t)n0 * p.ldb;
  auto issue = [&](int s) {
    const uint32_t base = smem_addr + (s % GEMM_NBUF) * GEMM_STAGE_BYTES;
    const int64_t k0 = (int64_t)min(s, p.K / GEMM_BK - 1) * GEMM_BK;  // past the end: a duplicate
#pragma unroll
    for (int q = 0; q < GEMM_LPW; ++q)
      tsp_lds_dma16((dma_isb[q] ? b_tile : a_tile) + k0, dma_voff[q], base + dma_slot[q]);
  };

  // operand reads: block rows (32 of them) `col`, logical chunk 2kk + half of the 16-k step
  int aoff[2], boff[2];  // byte offsets of rows 32*bi + col within the A (m) / B (n) tiles
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    aoff[bi] = (64 * wm + 32 * bi + col) * 128;
    boff[bi] = GEMM_TILE_BYTES + (64 * wn + 32 * bi + col) * 128;
  }
  const int rsw_a[2] = {gemm_swz(64 * wm + col), gemm_swz(64 * wm + 32 + col)};
  const int rsw_b[2] = {gemm_swz(64 * wn + col), gemm_swz(64 * wn + 32 + col)};

  tsp_f32x16 acc[2][2];  // [n block][m block]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

  const int n_stages = p.K / GEMM_BK;
  issue(0);
#pragma unroll 1
  for (int s = 0; s < n_stages; ++s) {
    tsp_wait_vm<0>();  // stage s landed (this wave's part)
    __syncthreads();   // ... for every wave; every wave is done with stage s-1
    issue(s + 1);      // into the other slot (past the end: a duplicate, drained below)
    const uint8_t* st = smem + (s % GEMM_NBUF) * GEMM_STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < GEMM_BK / 16; ++kk) {
      tsp_bf16x8 av[2], bv[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        av[bi] = __builtin_bit_cast(
            tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st + aoff[bi] + (((2 * kk + half) ^ rsw_a[bi]) << 4)));
        bv[bi] = __builtin_bit_cast(
            tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(st + boff[bi] + (((2 * kk + half) ^ rsw_b[bi]) << 4)));
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[x], av[y], acc[x][y], 0, 0, 0);
    }
  }
  tsp_wait_vm<0>();

  // epilogue: lane holds row m = m0 + 64wm + 32y + col, columns n0 + 64wn + 32x + 8a + 4half + 0..3
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int32_t m = m0 + 64 * wm + 32 * y + col;
    if (m >= p.M) continue;
    int64_t orow = m;
    if (p.zigzag) {
      const int32_t bb = m / p.S_local, i = m - bb * p.S_local;
      orow = (int64_t)bb * p.S_total + tsp_zigzag_position(i, p.C, p.D, p.rank);
    }
    const int64_t rbase = orow * p.ldc + p.c_col;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int32_t n = n0 + 64 * wn + 32 * x + 8 * a + 4 * half;
        if (n >= p.N) continue;  // N is a multiple of 4: a quad is either in or out
        const float v0 = acc[x][y][4 * a], v1 = acc[x][y][4 * a + 1], v2 = acc[x][y][4 * a + 2],
                    v3 = acc[x][y][4 * a + 3];
        if (p.mode == GEMM_STORE_BF16) {
          *reinterpret_cast<tsp_u32x2*>(static_cast<uint16_t*>(p.c) + rbase + n) =
              tsp_u32x2{tsp_pack_bf16(v0, v1), tsp_pack_bf16(v2, v3)};
        } else {
          float4* cp = reinterpret_cast<float4*>(static_cast<float*>(p.c) + rbase + n);
          float4 r = make_float4(v0, v1, v2, v3);
          if (p.mode != GEMM_STORE_F32) {
            const float4 o = *cp;
            r = make_float4(o.x + v0, o.y + v1, o.z + v2, o.w + v3);
          }
          if (p.mode == GEMM_ADD_F32_TO_BF16)
            *reinterpret_cast<tsp_u32x2*>(static_cast<uint16_t*>(p.c2) + rbase + n) =
                tsp_u32x2{tsp_pack_bf16(r.x, r.y), tsp_pack_bf16(r.z, r.w)};
          else
            *cp = r;
        }
      }
  }
}

}  // namespace tsp
