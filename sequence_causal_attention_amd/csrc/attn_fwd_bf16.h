// attn_fwd_bf16.h -- causal attention forward of one sequence-parallel rank, bf16 in,
// fp32 accumulation, bf16 MFMA (v_mfma_f32_32x32x16_bf16) for both products.
//
// What is computed ("Folding Tensor and Sequence Parallelism ...", section 2, attention
// layers; "AutoSP ...", section 2.A item 4; "Tensor, pipeline e sequence parallelism",
// section 01, GQA paragraph): for each local query row i of the rank and query head h,
// softmax over the keys j <= g(i) of the scaled scores q_i . k_j / sqrt(dh), applied to
// the values of KV head h / grp; plus lse_i, the natural-log log-sum-exp of the scores.
//
// Work decomposition (MI355X-specific, not from the pages):
//  * A workgroup owns one KV head, GH of its query heads, and a pair of query tiles of BQ
//    local rows: tile n_qtiles-1-p and tile p. Under the zigzag map the two tiles of a
//    pair need (2D*C + BQ) keys together whatever p and the rank, so every workgroup
//    does the same work and no rank is slower than another.
//  * Every wave owns RB row blocks of 32 query rows (32 consecutive local rows of one
//    head). Scores are computed transposed, S^T = K Q^T (keys along MFMA rows, queries
//    along MFMA columns), so each lane holds one query column: the row max and row sum
//    are in-lane except for one exchange between the two 32-lane halves, and the fp32
//    score accumulator, rounded to bf16, is already the B operand of O^T = V^T P^T.
//  * K and V tiles of BK keys are staged once per workgroup in LDS and shared by all
//    waves, hence by all GH query heads of the KV group; the next tile's global loads
//    are in flight while the current tile is being computed (double buffer, one
//    barrier per tile). V is transposed while it is written to LDS, its keys placed in
//    the order the P operand holds them, so every MFMA operand is one 16-byte LDS read.
//  * KV tiles past the query tile's last global position are never loaded (causal tile
//    skipping); only tiles that cross a wave's first position are masked element-wise,
//    by comparing the key index with the query's global position.
//  * Online softmax in the base-2 domain (log2(e)/sqrt(dh) folded into one FMA) with a
//    lazily raised running max (see TSP_RESCALE_SLACK).
#pragma once

#include "attn_common.h"

namespace tsp {

template <int DH, int BK>
struct Bf16Tile {
  static constexpr int KP = DH + 8;          // K tile row pitch (elements): conflict-free 16 B reads
  static constexpr int VP = BK + 8;          // V^T tile row pitch (elements)
  static constexpr int K_ELEMS = BK * KP;
  static constexpr int V_ELEMS = DH * VP;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BK * DH / 8;        // 16-byte pieces of a K tile
  static constexpr int V_GROUPS = (BK / 4) * (DH / 8);  // (4 keys x 8 dims) pieces of a V tile
};

// LDS column of the first key of 4-key group `kg` inside a V^T row. Within each block of
// 32 keys, key 8a + 4h + b (a < 4, h < 2, b < 4) goes to column 16(a/2) + 8h + 4(a%2) + b:
// the 8 keys a lane half h feeds to one PV MFMA step become 8 contiguous columns.
__device__ __forceinline__ int tsp_vt_group_col(int kg) {
  const int blk = kg >> 3, g = kg & 7, a = g >> 1, h = g & 1;
  return blk * 32 + 16 * (a >> 1) + 8 * h + 4 * (a & 1);
}

template <int DH, int BK, int NW, int RB>
__global__ __launch_bounds__(NW * 64) void attn_fwd_bf16_kernel(TspParams p) {
  using T = Bf16Tile<DH, BK>;
  constexpr int NT = NW * 64;
  constexpr int NKC = (T::K_CHUNKS + NT - 1) / NT;
  constexpr int NVG = (T::V_GROUPS + NT - 1) / NT;
  constexpr int NKB = BK / 32;  // 32-key blocks per tile
  constexpr int NDB = DH / 32;  // 32-dim blocks of the output
  static_assert(BK % 32 == 0 && DH % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  const int64_t kv_row_stride = (int64_t)p.Hkv * DH;  // elements between consecutive keys
  const uint16_t* __restrict__ kbase = kg + ((int64_t)b * p.S_total * p.Hkv + hk) * DH;
  const uint16_t* __restrict__ vbase = vg + ((int64_t)b * p.S_total * p.Hkv + hk) * DH;

  const int pos_blocks = p.BQ / 32;  // row blocks per head in a tile

  for (int which = 0; which < 2; ++which) {
    const int32_t qt = which == 0 ? p.n_qtiles - 1 - pair : pair;
    if (which == 1 && qt == p.n_qtiles - 1 - pair) break;  // middle tile of an odd count
    const int32_t row0 = qt * p.BQ;
    const int32_t last_row = min(row0 + p.BQ, p.S_local) - 1;
    const int32_t kv_end = tsp_zigzag_position(last_row, p.C, p.D, p.rank) + 1;
    const int32_t n_kv = (kv_end + BK - 1) / BK;

    // ---- this wave's query rows -------------------------------------------------------
    int32_t lrow[RB], qpos[RB], head[RB];
    bool rvalid[RB];
    int32_t wave_first = 0x7fffffff, wave_last = -1;  // local rows (uniform)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rbi = wave * RB + rb;
      const int pb = rbi % pos_blocks, hh = rbi / pos_blocks;
      head[rb] = hk * p.grp + hgrp * p.GH + hh;
      const int32_t r = row0 + pb * 32 + col;
      rvalid[rb] = r < p.S_local;
      lrow[rb] = min(r, p.S_local - 1);
      qpos[rb] = tsp_zigzag_position(lrow[rb], p.C, p.D, p.rank);
      wave_first = min(wave_first, row0 + pb * 32);
      wave_last = max(wave_last, min(row0 + pb * 32 + 31, p.S_local - 1));
    }
    const bool wave_active = wave_first < p.S_local;
    const int32_t wave_min_pos = tsp_zigzag_position(min(wave_first, p.S_local - 1), p.C, p.D, p.rank);
    const int32_t wave_max_pos = tsp_zigzag_position(wave_last, p.C, p.D, p.rank);

    // ---- Q^T operands stay in registers for the whole sweep -----------------------------
    tsp_bf16x8 qf[RB][DH / 16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint16_t* qp = qg + (((int64_t)b * p.S_local + lrow[rb]) * p.Hq + head[rb]) * DH + half * 8;
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk)
        qf[rb][kk] = __builtin_bit_cast(tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(qp + kk * 16));
    }

    tsp_f32x16 acc[RB][NDB];
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m_run[rb] = -INFINITY;
      l_run[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][db][e] = 0.f;
    }

    // ---- staging of one K/V tile: global -> registers -> LDS ----------------------------
    tsp_u32x4 kreg[NKC];
    tsp_u32x4 vreg[NVG][4];
    auto load_tile = [&](int j) {
      const int32_t kv0 = j * BK;
#pragma unroll
      for (int it = 0; it < NKC; ++it) {
        const int c = tid + it * NT;
        const int row = c / (DH / 8), c8 = c % (DH / 8);
        const int32_t key = kv0 + row;
        tsp_u32x4 z = {0u, 0u, 0u, 0u};
        if ((T::K_CHUNKS % NT == 0 || c < T::K_CHUNKS) && key < kv_end)
          z = *reinterpret_cast<const tsp_u32x4*>(kbase + key * kv_row_stride + c8 * 8);
        kreg[it] = z;
      }
#pragma unroll
      for (int it = 0; it < NVG; ++it) {
        const int g = tid + it * NT;
        const int kgp = g % (BK / 4), dc = g / (BK / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t key = kv0 + kgp * 4 + r;
          tsp_u32x4 z = {0u, 0u, 0u, 0u};
          if ((T::V_GROUPS % NT == 0 || g < T::V_GROUPS) && key < kv_end)
            z = *reinterpret_cast<const tsp_u32x4*>(vbase + key * kv_row_stride + dc * 8);
          vreg[it][r] = z;
        }
      }
    };
    auto store_tile = [&](int buf) {
      uint16_t* sk = smem + buf * T::STAGE;
      uint16_t* sv = sk + T::K_ELEMS;
#pragma unroll
      for (int it = 0; it < NKC; ++it) {
        const int c = tid + it * NT;
        if (T::K_CHUNKS % NT == 0 || c < T::K_CHUNKS) {
          const int row = c / (DH / 8), c8 = c % (DH / 8);
          *reinterpret_cast<tsp_u32x4*>(sk + row * T::KP + c8 * 8) = kreg[it];
        }
      }
#pragma unroll
      for (int it = 0; it < NVG; ++it) {
        const int g = tid + it * NT;
        if (T::V_GROUPS % NT == 0 || g < T::V_GROUPS) {
          const int kgp = g % (BK / 4), dc = g / (BK / 4);
          const int colv = tsp_vt_group_col(kgp);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int w = c >> 1;
            uint32_t x0 = vreg[it][0][w], x1 = vreg[it][1][w], x2 = vreg[it][2][w], x3 = vreg[it][3][w];
            tsp_u32x2 pk;
            if (c & 1) {
              pk[0] = (x0 >> 16) | (x1 & 0xffff0000u);
              pk[1] = (x2 >> 16) | (x3 & 0xffff0000u);
            } else {
              pk[0] = (x0 & 0xffffu) | (x1 << 16);
              pk[1] = (x2 & 0xffffu) | (x3 << 16);
            }
            *reinterpret_cast<tsp_u32x2*>(sv + (dc * 8 + c) * T::VP + colv) = pk;
          }
        }
      }
    };

    __syncthreads();  // the previous tile's last readers are done with both buffers
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_kv; ++j) {
      const bool more = j + 1 < n_kv;
      if (more) load_tile(j + 1);
      const int32_t kv0 = j * BK;

      if (wave_active && kv0 <= wave_max_pos) {
        const uint16_t* sk = smem + (j & 1) * T::STAGE;
        const uint16_t* sv = sk + T::K_ELEMS;

        // S^T = K Q^T for this tile: NKB blocks of 32 keys x 32 queries per row block.
        tsp_f32x16 s[RB][NKB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[rb][kb][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < DH / 16; ++kk) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const tsp_bf16x8 kf = __builtin_bit_cast(
                tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(sk + (kb * 32 + col) * T::KP + kk * 16 + half * 8));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              s[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][kk], s[rb][kb], 0, 0, 0);
          }
        }

        // Mask, online softmax, P^T operands.
        const bool need_mask = kv0 + BK - 1 > wave_min_pos;
        tsp_bf16x8 pf[RB][BK / 16];
    #pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
          // lane holds keys kv0 + 32kb + 8(e/4) + 4*half + (e%4) of query column `col`
          const int32_t lim = qpos[rb] - kv0 - 4 * half;
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float x = s[rb][kb][e];
              if (need_mask && (kb * 32 + 8 * (e >> 2) + (e & 3)) > lim) x = -INFINITY;
              s[rb][kb][e] = x;
              mx = fmaxf(mx, x);
            }
          mx = tsp_max_halves(mx);
          const float mt = mx * p.scale_log2;
          if (__builtin_amdgcn_ballot_w64(mt > m_run[rb] + TSP_RESCALE_SLACK) != 0) {
            const float m_new = fmaxf(m_run[rb], mt);
            const float alpha = tsp_exp2(m_run[rb] - m_new);
            m_run[rb] = m_new;
            l_run[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[rb][db][e] *= alpha;
          }
          const float mneg = -m_run[rb];
          float lsum = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              float pv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) pv[e] = tsp_exp2(fmaf(s[rb][kb][st * 8 + e], p.scale_log2, mneg));
              tsp_u32x4 w;
              w[0] = tsp_pack_bf16(pv[0], pv[1]);
              w[1] = tsp_pack_bf16(pv[2], pv[3]);
              w[2] = tsp_pack_bf16(pv[4], pv[5]);
              w[3] = tsp_pack_bf16(pv[6], pv[7]);
              // the row sum uses the rounded weights the PV product applies
#pragma unroll
              for (int e = 0; e < 4; ++e) lsum = tsp_sum_bf16_pair(w[e], lsum);
              pf[rb][kb * 2 + st] = __builtin_bit_cast(tsp_bf16x8, w);
            }
          }
          l_run[rb] += lsum;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int st = 0; st < BK / 16; ++st) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const tsp_bf16x8 vf = __builtin_bit_cast(
                tsp_bf16x8, *reinterpret_cast<const tsp_u32x4*>(sv + (db * 32 + col) * T::VP + st * 16 + half * 8));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb][st], acc[rb][db], 0, 0, 0);
          }
        }
      }

      if (more) store_tile((j + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue: normalise, round to bf16, write O and lse -----------------------------
    if (wave_active) {
  #pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l = tsp_sum_halves(l_run[rb]);
        const float inv = 1.0f / l;
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
                (m_run[rb] + __builtin_amdgcn_logf(l)) * TSP_LN2;
        }
      }
    }
  }
}

}  // namespace tsp
