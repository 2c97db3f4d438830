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
#ifndef TSP_BWD_KV_PIPE_DV
#define TSP_BWD_KV_PIPE_DV 1  // the dV launch has the registers for it (188 VGPRs)
#endif
#ifndef TSP_BWD_KV_PIPE_DK
#define TSP_BWD_KV_PIPE_DK TSP_BWD_KV_PIPE
#endif
#ifndef TSP_BWD_Q_NW
#define TSP_BWD_Q_NW 8
#endif
#ifndef TSP_BWD_KV_NW_DV
#define TSP_BWD_KV_NW_DV 4
#endif
#ifndef TSP_BWD_KV_NW_DK
#define TSP_BWD_KV_NW_DK 4
#endif
#ifndef TSP_BWD_KV_SPLIT
#define TSP_BWD_KV_SPLIT 1
#endif
#ifndef TSP_BWD_KV_FUSED
#define TSP_BWD_KV_FUSED 1
#endif
#ifndef TSP_BWD_KV_NW_FUSED
#define TSP_BWD_KV_NW_FUSED 8
#endif
#ifndef TSP_BWD_KV_NBUF_FUSED
#define TSP_BWD_KV_NBUF_FUSED 4
#endif
template <int DH>
struct BwdCfg {
  static constexpr int KV_NW = 4, KV_NBUF = DH <= 128 ? TSP_BWD_KV_NBUF : 4;
  static constexpr int KV_NW_DV = DH <= 128 ? TSP_BWD_KV_NW_DV : KV_NW;  // waves of the dV launch
  static constexpr int KV_NW_DK = DH <= 128 ? TSP_BWD_KV_NW_DK : KV_NW;  // waves of the dK launch
  static constexpr bool KV_PIPE = DH <= 128 && TSP_BWD_KV_PIPE;
  static constexpr bool KV_PIPE_DV = DH <= 128 && TSP_BWD_KV_PIPE_DV, KV_PIPE_DK = DH <= 128 && TSP_BWD_KV_PIPE_DK;
  // with the one-launch form off: dK and dV in separate launches at two waves per SIMD
  // (dh <= 128), or one launch at one wave per SIMD
  static constexpr bool KV_SPLIT = DH <= 128 && TSP_BWD_KV_SPLIT;
  // dK and dV in one launch at two waves per SIMD, V parked in LDS (dh <= 128)
  static constexpr bool KV_FUSED = DH <= 128 && TSP_BWD_KV_FUSED;
  static constexpr int KV_NW_FUSED = TSP_BWD_KV_NW_FUSED, KV_NBUF_FUSED = TSP_BWD_KV_NBUF_FUSED;
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
  if constexpr (C::KV_FUSED) {
    tsp::TspBwdParams bf = bp;
    bf.n_kblocks = (bp.f.S_total + 32 * C::KV_NW_FUSED - 1) / (32 * C::KV_NW_FUSED);
    const int64_t f_units = kv_units / bp.n_kblocks * bf.n_kblocks;
    hipLaunchKernelGGL(
        (tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW_FUSED, C::KV_NBUF_FUSED, false, tsp::BWD_KV_BOTH, 2, true>),
        dim3((unsigned)f_units), dim3(C::KV_NW_FUSED * 64), 0, s, bf);
  } else if constexpr (C::KV_SPLIT) {
    // the dV launch may own more keys per workgroup: its own key blocks
    tsp::TspBwdParams bv = bp;
    bv.n_kblocks = (bp.f.S_total + 32 * C::KV_NW_DV - 1) / (32 * C::KV_NW_DV);
    const int64_t dv_units = kv_units / bp.n_kblocks * bv.n_kblocks;
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW_DV, C::KV_NBUF, C::KV_PIPE_DV, tsp::BWD_KV_DV, 2>),
                       dim3((unsigned)dv_units), dim3(C::KV_NW_DV * 64), 0, s, bv);
    tsp::TspBwdParams bk = bp;
    bk.n_kblocks = (bp.f.S_total + 32 * C::KV_NW_DK - 1) / (32 * C::KV_NW_DK);
    const int64_t dk_units = kv_units / bp.n_kblocks * bk.n_kblocks;
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW_DK, C::KV_NBUF, C::KV_PIPE_DK, tsp::BWD_KV_DK, 2>),
                       dim3((unsigned)dk_units), dim3(C::KV_NW_DK * 64), 0, s, bk);
  } else {
    hipLaunchKernelGGL((tsp::attn_bwd_dkv_bf16_kernel<DH, C::KV_NW, C::KV_NBUF, C::KV_PIPE, tsp::BWD_KV_BOTH, 1>),
                       dim3((unsigned)kv_units), dim3(C::KV_NW * 64), 0, s, bp);
  }
}

