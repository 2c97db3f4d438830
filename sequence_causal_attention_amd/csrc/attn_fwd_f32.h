// attn_fwd_f32.h -- the same per-rank causal attention for float32 inputs, with fp32
// MFMA (v_mfma_f32_32x32x2_f32) products and fp32 accumulation.
//
// Same definition, work decomposition, transposed-score layout, masking and online
// softmax as the bf16 kernel (attn_fwd_bf16.h); the differences are the operand width
// (one fp32 value per lane per MFMA, 2 reduction steps per instruction), P kept in fp32,
// and a single LDS buffer with K and V both row-major (V is read one value per lane, so
// no transposed copy is needed). It serves small fp32 shards; speed is not its purpose.
#pragma once

#include "attn_common.h"

namespace tsp {

template <int DH>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(TspParams p) {
  constexpr int NW = 4, NT = NW * 64, BK = 32;
  constexpr int KP = DH + 1;  // row pitch (floats) of the K and V tiles
  constexpr int CHUNKS = BK * DH / 4;  // 16-byte pieces of a tile
  constexpr int NC = CHUNKS / NT;
  constexpr int NDB = DH / 32;
  static_assert(CHUNKS % NT == 0, "tile shape");

  __shared__ float sk[BK * KP];
  __shared__ float sv[BK * KP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  const float* __restrict__ qg = static_cast<const float*>(p.q);
  const float* __restrict__ kg = static_cast<const float*>(p.k);
  const float* __restrict__ vg = static_cast<const float*>(p.v);
  float* __restrict__ og = static_cast<float*>(p.out);

  int32_t unit = tsp_xcd_unit(blockIdx.x, gridDim.x);
  const int32_t pair = unit % p.n_pairs;
  unit /= p.n_pairs;
  const int32_t hgrp = unit % p.n_hgroups;
  unit /= p.n_hgroups;
  const int32_t hk = unit % p.Hkv;
  const int32_t b = unit / p.Hkv;

  const int64_t kv_row_stride = p.kv_stride;
  const float* __restrict__ kbase = kg + (int64_t)b * p.S_total * p.kv_stride + (int64_t)hk * DH;
  const float* __restrict__ vbase = vg + (int64_t)b * p.S_total * p.kv_stride + (int64_t)hk * DH;
  const int pos_blocks = p.BQ / 32;

  for (int which = 0; which < 2; ++which) {
    const int32_t qt = which == 0 ? p.n_qtiles - 1 - pair : pair;
    if (which == 1 && qt == p.n_qtiles - 1 - pair) break;
    const int32_t row0 = qt * p.BQ;
    const int32_t last_row = min(row0 + p.BQ, p.S_local) - 1;
    // keys [kv_lo, kv_end) take part: up to the tile's last position, or the range end
    const int32_t kv_end = min(p.kv_hi, tsp_zigzag_position(last_row, p.C, p.D, p.rank) + 1);
    const int32_t j0 = p.kv_lo / BK;  // first key tile of the range
    const int32_t n_kv = (kv_end + BK - 1) / BK;

    const int pb = wave % pos_blocks, hh = wave / pos_blocks;
    const int32_t head = hk * p.grp + hgrp * p.GH + hh;
    const int32_t first = row0 + pb * 32;
    const int32_t r = first + col;
    const bool rvalid = r < p.S_local;
    const int32_t lrow = min(r, p.S_local - 1);
    // last visible key of the row: its position, or the range end if that comes first
    const int32_t qpos = min(tsp_zigzag_position(lrow, p.C, p.D, p.rank), p.kv_hi - 1);
    const bool wave_active = first < p.S_local;
    const int32_t wave_min_pos = tsp_zigzag_position(min(first, p.S_local - 1), p.C, p.D, p.rank);
    const int32_t wave_max_pos = tsp_zigzag_position(min(first + 31, p.S_local - 1), p.C, p.D, p.rank);

    // Q^T operand: lane holds q[row col][2kk + half] for every reduction step kk.
    float qf[DH / 2];
    const float* qp = qg + (((int64_t)b * p.S_local + lrow) * p.Hq + head) * DH + half;
#pragma unroll
    for (int kk = 0; kk < DH / 2; ++kk) qf[kk] = qp[2 * kk];

    tsp_f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int j = j0; j < n_kv; ++j) {
      const int32_t kv0 = j * BK;
      __syncthreads();  // previous tile fully consumed
#pragma unroll
      for (int it = 0; it < NC; ++it) {
        const int c = tid + it * NT;
        const int row = c / (DH / 4), c4 = c % (DH / 4);
        const int32_t key = kv0 + row;
        float4 kz = make_float4(0.f, 0.f, 0.f, 0.f), vz = kz;
        if (key < kv_end) {
          kz = *reinterpret_cast<const float4*>(kbase + key * kv_row_stride + c4 * 4);
          vz = *reinterpret_cast<const float4*>(vbase + key * kv_row_stride + c4 * 4);
        }
        float* dk = sk + row * KP + c4 * 4;
        float* dv = sv + row * KP + c4 * 4;
        dk[0] = kz.x; dk[1] = kz.y; dk[2] = kz.z; dk[3] = kz.w;
        dv[0] = vz.x; dv[1] = vz.y; dv[2] = vz.z; dv[3] = vz.w;
      }
      __syncthreads();
      if (!wave_active || kv0 > wave_max_pos) continue;

      // S^T = K Q^T (32 keys x 32 queries)
      tsp_f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < DH / 2; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(sk[col * KP + 2 * kk + half], qf[kk], s, 0, 0, 0);

      // lane holds keys kv0 + 8(e/4) + 4*half + (e%4) of query column `col`: visible iff
      // <= qpos and >= kv_lo
      const bool need_mask = kv0 + BK - 1 > min(wave_min_pos, p.kv_hi - 1) || kv0 < p.kv_lo;
      const int32_t hi = qpos - kv0 - 4 * half;
      const int32_t lo = p.kv_lo - kv0 - 4 * half;
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[e];
        const int off = 8 * (e >> 2) + (e & 3);
        if (need_mask && (off > hi || off < lo)) x = -INFINITY;
        s[e] = x;
        mx = fmaxf(mx, x);
      }
      mx = tsp_max_halves(mx);
      const float mt = mx * p.scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + TSP_RESCALE_SLACK) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : tsp_exp2(m_run - m_new);  // still no visible key
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
      }
      const float mneg = m_run == -INFINITY ? 0.f : -m_run;  // no visible key yet: weights 0
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = tsp_exp2(fmaf(s[e], p.scale_log2, mneg));
        l_run += s[e];
      }

      // O^T += V^T P^T, one key per lane half per step: step e uses key 8(e/4)+4*half+(e%4)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int krow = 8 * (e >> 2) + 4 * half + (e & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sv[krow * KP + db * 32 + col], s[e], acc[db], 0, 0, 0);
      }
    }

    if (wave_active && p.accumulate) {  // merge this partial into the running result
      const float l = tsp_sum_halves(l_run);
      if (rvalid && l > 0.f) {
        float* lp = p.lse + ((int64_t)b * p.Hq + head) * p.S_local + lrow;
        float w_old, w_new;
        const float lse_new = tsp_merge_weights(*lp, m_run, l, w_old, w_new);
        float* op = og + (((int64_t)b * p.S_local + lrow) * p.Hq + head) * DH + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            float4* dst = reinterpret_cast<float4*>(op + db * 32 + 8 * a);
            const float4 o = *dst;
            *dst = make_float4(fmaf(w_new, acc[db][4 * a], w_old * o.x), fmaf(w_new, acc[db][4 * a + 1], w_old * o.y),
                               fmaf(w_new, acc[db][4 * a + 2], w_old * o.z),
                               fmaf(w_new, acc[db][4 * a + 3], w_old * o.w));
          }
        if (half == 0) *lp = lse_new;  // both halves read the old lse above
      }
    } else if (wave_active) {
      const float l = tsp_sum_halves(l_run);
      const float inv = l > 0.f ? 1.0f / l : 0.f;  // l = 0: no visible key in the range
      if (rvalid) {
        float* op = og + (((int64_t)b * p.S_local + lrow) * p.Hq + head) * DH + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *reinterpret_cast<float4*>(op + db * 32 + 8 * a) =
                make_float4(acc[db][4 * a] * inv, acc[db][4 * a + 1] * inv, acc[db][4 * a + 2] * inv,
                            acc[db][4 * a + 3] * inv);
        if (half == 0)
          p.lse[((int64_t)b * p.Hq + head) * p.S_local + lrow] =
              l > 0.f ? (m_run + __builtin_amdgcn_logf(l)) * TSP_LN2 : -INFINITY;
      }
    }
    __syncthreads();
  }
}

}  // namespace tsp
