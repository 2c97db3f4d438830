// attn_bwd_f32.h -- backward of the per-rank causal attention for float32 inputs: the
// same gradients as attn_bwd_bf16.h (delta, dQ, the rank's partial dK/dV), fp32 end to
// end. It serves small fp32 shards; speed is not its purpose.
//
// One wave per output vector, the head dim spread over the lanes (DH/64 values per
// lane), dot products reduced across the wave:
//  * dQ: a wave per (b, local row, query head) sweeps the keys j <= g(row);
//  * dK/dV: a wave per (b, key, KV head) sweeps the query heads of the group and the local
//    rows that see the key (rows are increasing in position, so they are a suffix of each
//    chunk).
#pragma once

#include "attn_common.h"
#include "attn_bwd_bf16.h"

namespace tsp {

__device__ __forceinline__ float tsp_wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_delta_f32_kernel(TspBwdParams p) {
  constexpr int TPR = DH / 4;  // threads per (row, head) vector, 16 bytes each
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = tid / TPR;
  const int c = (int)(tid % TPR);
  const bool valid = row < p.n_rows;
  float acc = 0.f;
  if (valid) {
    const float4 o = reinterpret_cast<const float4*>(static_cast<const float*>(p.f.out) + row * DH)[c];
    const float4 d = reinterpret_cast<const float4*>(static_cast<const float*>(p.dout) + row * DH)[c];
    acc = o.x * d.x + o.y * d.y + o.z * d.z + o.w * d.w;
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

template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32_kernel(TspBwdParams bp) {
  constexpr int E = DH / 64;  // dims per lane: lane l holds dims l + 64e
  const TspParams& p = bp.f;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (wid >= bp.n_rows) return;
  const int32_t h = (int32_t)(wid % p.Hq);
  const int64_t bi = wid / p.Hq;
  const int32_t i = (int32_t)(bi % p.S_local);
  const int64_t b = bi / p.S_local;
  const int32_t hk = h / p.grp;
  const int32_t pos = tsp_zigzag_position(i, p.C, p.D, p.rank);
  const float* qv = static_cast<const float*>(p.q) + wid * DH;
  const float* dov = static_cast<const float*>(bp.dout) + wid * DH;
  float q[E], dO[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qv[lane + 64 * e];
    dO[e] = dov[lane + 64 * e];
    acc[e] = 0.f;
  }
  const int64_t li = (b * p.Hq + h) * p.S_local + i;
  const float lse = p.lse[li], delta = bp.delta[li];
  const int64_t kv_row = (int64_t)p.Hkv * DH;
  const float* kb = static_cast<const float*>(p.k) + b * p.S_total * kv_row + (int64_t)hk * DH;
  const float* vb = static_cast<const float*>(p.v) + b * p.S_total * kv_row + (int64_t)hk * DH;
  for (int32_t j = 0; j <= pos; ++j) {
    float s = 0.f, dp = 0.f, kj[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kj[e] = kb[j * kv_row + lane + 64 * e];
      s = fmaf(q[e], kj[e], s);
      dp = fmaf(dO[e], vb[j * kv_row + lane + 64 * e], dp);
    }
    s = tsp_wave_sum(s);
    dp = tsp_wave_sum(dp);
    const float pj = __expf(s * bp.scale - lse);
    const float ds = pj * (dp - delta);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kj[e], acc[e]);
  }
  float* dq = static_cast<float*>(bp.dq) + wid * DH;
#pragma unroll
  for (int e = 0; e < E; ++e) dq[lane + 64 * e] = acc[e] * bp.scale;
}

template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_dkv_f32_kernel(TspBwdParams bp) {
  constexpr int E = DH / 64;
  const TspParams& p = bp.f;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (wid >= bp.n_kv_rows) return;
  const int32_t hk = (int32_t)(wid % p.Hkv);
  const int64_t bj = wid / p.Hkv;
  const int32_t j = (int32_t)(bj % p.S_total);
  const int64_t b = bj / p.S_total;
  const int64_t kv_row = (int64_t)p.Hkv * DH;
  const int64_t koff = (b * p.S_total + j) * kv_row + (int64_t)hk * DH;
  float kj[E], vj[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kj[e] = static_cast<const float*>(p.k)[koff + lane + 64 * e];
    vj[e] = static_cast<const float*>(p.v)[koff + lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  // local rows that see key j: a suffix of each chunk
  const int32_t C = p.C;
  const int32_t a0 = min(C, max(0, j - p.rank * C));                           // first chunk
  const int32_t b0 = C + min(C, max(0, j - (2 * p.D - 1 - p.rank) * C));     // second chunk
  for (int32_t g = 0; g < p.grp; ++g) {
    const int32_t h = hk * p.grp + g;
    for (int part = 0; part < 2; ++part) {
      const int32_t r_begin = part == 0 ? a0 : b0, r_end = part == 0 ? C : 2 * C;
      for (int32_t i = r_begin; i < r_end; ++i) {
        const int64_t qo = ((b * p.S_local + i) * p.Hq + h) * DH;
        const float* qv = static_cast<const float*>(p.q) + qo;
        const float* dov = static_cast<const float*>(bp.dout) + qo;
        float s = 0.f, dp = 0.f, qi[E], doi[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          qi[e] = qv[lane + 64 * e];
          doi[e] = dov[lane + 64 * e];
          s = fmaf(qi[e], kj[e], s);
          dp = fmaf(doi[e], vj[e], dp);
        }
        s = tsp_wave_sum(s);
        dp = tsp_wave_sum(dp);
        const int64_t li = (b * p.Hq + h) * p.S_local + i;
        const float pij = __expf(s * bp.scale - p.lse[li]);
        const float ds = pij * (dp - bp.delta[li]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dv[e] = fmaf(pij, doi[e], dv[e]);
          dk[e] = fmaf(ds, qi[e], dk[e]);
        }
      }
    }
  }
  float* dkp = static_cast<float*>(bp.dk) + koff;
  float* dvp = static_cast<float*>(bp.dv) + koff;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dkp[lane + 64 * e] = dk[e] * bp.scale;
    dvp[lane + 64 * e] = dv[e];
  }
}

}  // namespace tsp
