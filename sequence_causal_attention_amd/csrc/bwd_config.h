// bwd_config.h -- tile configuration and launch entry of the backward kernels, shared by
// the backward translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_bwd_bf16.h"

// Tile configuration per head dim: waves of the key-stationary and query-stationary
// kernels, their LDS ring depths, and the query-stationary kernel's waves per SIMD.
#ifndef TSP_BWD_KV_NBUF
#define TSP_BWD_KV_NBUF 4
#endif
#ifndef TSP_BWD_KV_PIPE
#define TSP_BWD_KV_PIPE 0
#endif
#ifndef TSP_BWD_Q_NW
#define TSP_BWD_Q_NW 8
#endif
#ifndef TSP_BWD_KV_SPLIT
#define TSP_BWD_KV_SPLIT 1
#endif
template <int DH>
struct BwdCfg {
  static constexpr int KV_NW = 4, KV_NBUF = DH <= 128 ? TSP_BWD_KV_NBUF : 4;
  static constexpr bool KV_PIPE = DH <= 128 && TSP_BWD_KV_PIPE;
  // dK and dV in separate launches at two waves per SIMD (dh <= 128), or one launch
  static constexpr bool KV_SPLIT = DH <= 128 && TSP_BWD_KV_SPLIT;
  static constexpr int Q_NW = DH <= 128 ? TSP_BWD_Q_NW : 4, Q_NBUF = 4, Q_OCC = DH <= 128 ? 2 : 1;
};

// The kernels of one head dim, in the order delta, dQ, dK/dV. Instantiated for dh 64 and
// 128 in tsp_attn_bwd.hip and for dh 256 in tsp_attn_bwd256.hip.
template <int DH>
void tsp_bwd_launch(const tsp::TspBwdParams& bp, int64_t kv_units, hipStream_t s) {
  using C = BwdCfg<DH>;
  const int64_t threads = bp.n_rows * (DH / 8);
  hipLaunchKernelGGL((tsp::attn_bwd_delta_bf16_kernel<DH>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, bp);
  hipLaunchKernelGGL((tsp::attn_bwd_dq_bf16_kernel<DH, C::Q_NW, C::Q_NBUF, C::Q_OCC>), dim3(bp.f.n_units),
                     dim3(C::Q_NW * 64), 0, s, bp);
  if constexpr (C::KV_SPLIT) {
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW, C::KV_NBUF, C::KV_PIPE, tsp::BWD_KV_DV, 2>),
                       dim3((unsigned)kv_units), dim3(C::KV_NW * 64), 0, s, bp);
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW, C::KV_NBUF, C::KV_PIPE, tsp::BWD_KV_DK, 2>),
                       dim3((unsigned)kv_units), dim3(C::KV_NW * 64), 0, s, bp);
  } else {
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW, C::KV_NBUF, C::KV_PIPE, tsp::BWD_KV_BOTH, 1>),
                       dim3((unsigned)kv_units), dim3(C::KV_NW * 64), 0, s, bp);
  }
}

