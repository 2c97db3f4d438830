// tsp_attn_bwd.hip -- C ABI of the backward of the per-rank zigzag / GQA causal attention
// (gfx950): argument validation, work decomposition and dispatch of the three backward
// kernels (attn_bwd_bf16.h).
#include <hip/hip_runtime.h>

#include "tsp_attn.h"
#include "attn_bwd_bf16.h"
#include "host_common.h"
#include "bwd_config.h"
#include "attn_bwd_f32.h"

namespace {

using tsp_host::aligned16;
using tsp_host::fail;
using tsp_host::KernelShape;

}  // namespace

template void tsp_bwd_launch<64>(const tsp::TspBwdParams&, int64_t, hipStream_t);
template void tsp_bwd_launch<128>(const tsp::TspBwdParams&, int64_t, hipStream_t);
// dh 256 is instantiated in tsp_attn_bwd256.hip (built with other code-generation flags)
extern template void tsp_bwd_launch<256>(const tsp::TspBwdParams&, int64_t, hipStream_t);

namespace {

template <int DH>
void launch_f32(const tsp::TspBwdParams& bp, hipStream_t s) {
  const int64_t threads = bp.n_rows * (DH / 4);
  hipLaunchKernelGGL((tsp::attn_bwd_delta_f32_kernel<DH>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     bp);
  hipLaunchKernelGGL((tsp::attn_bwd_dq_f32_kernel<DH>), dim3((unsigned)((bp.n_rows + 3) / 4)), dim3(256), 0, s, bp);
  hipLaunchKernelGGL((tsp::attn_bwd_dkv_f32_kernel<DH>), dim3((unsigned)((bp.n_kv_rows + 3) / 4)), dim3(256), 0, s,
                     bp);
}

template <int DH>
int kv_block() {
  return 32 * BwdCfg<DH>::KV_NW;
}

}  // namespace

extern "C" {

int tsp_attn_bwd(const void* q_local, const void* k_full, const void* v_full, const void* out, const float* lse,
                 const void* dout, void* dq_local, void* dk_full, void* dv_full, float* delta, int64_t B,
                 int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
                 void* stream) {
  const void* ptrs[] = {q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full, delta};
  for (const void* ptr : ptrs) {
    if (!ptr) return fail(TSP_EINVAL, "null pointer argument");
    if (!aligned16(ptr)) return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  }
  int st = tsp_host::check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (dtype != TSP_BF16 && dtype != TSP_F32) return fail(TSP_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (dh != 64 && dh != 128 && dh != 256)
    return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
  if (Hq >= 1 && Hq * dh > (int64_t(1) << 22)) return fail(TSP_EINVAL, "Hq * dh above 2^22");

  tsp::TspBwdParams bp{};
  const KernelShape ks{32, dh == 64 ? BwdCfg<64>::Q_NW : dh == 128 ? BwdCfg<128>::Q_NW : BwdCfg<256>::Q_NW, 1};
  st = tsp_host::plan_tiles(B, S_total, D, rank, Hq, Hkv, dh, ks, &bp.f);
  if (st != TSP_OK) return st;
  const int kb = dh == 64 ? kv_block<64>() : dh == 128 ? kv_block<128>() : kv_block<256>();
  const int64_t n_kblocks = (S_total + kb - 1) / kb;
  const int64_t kv_units = B * Hkv * n_kblocks;
  if (kv_units > 0x7fffffff) return fail(TSP_EINVAL, "problem too large for one launch");

  bp.f.q = q_local;
  bp.f.k = k_full;
  bp.f.v = v_full;
  bp.f.out = const_cast<void*>(out);
  bp.f.lse = const_cast<float*>(lse);
  bp.dout = dout;
  bp.dq = dq_local;
  bp.dk = dk_full;
  bp.dv = dv_full;
  bp.delta = delta;
  bp.n_rows = B * (int64_t)bp.f.S_local * Hq;
  bp.n_kv_rows = B * S_total * Hkv;
  if (dtype == TSP_F32 && (bp.n_rows > (int64_t(1) << 33) || bp.n_kv_rows > (int64_t(1) << 33)))
    return fail(TSP_EINVAL, "problem too large for the fp32 backward");
  bp.kv_need = (int32_t)((2 * D - rank) * bp.f.C);
  bp.n_kblocks = (int32_t)n_kblocks;
  bp.scale = (float)(1.0 / std::sqrt((double)dh));

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == TSP_F32) {
    switch (dh) {
      case 64: launch_f32<64>(bp, s); break;
      case 128: launch_f32<128>(bp, s); break;
      case 256: launch_f32<256>(bp, s); break;
    }
  } else {
    switch (dh) {
      case 64: tsp_bwd_launch<64>(bp, kv_units, s); break;
      case 128: tsp_bwd_launch<128>(bp, kv_units, s); break;
      case 256: tsp_bwd_launch<256>(bp, kv_units, s); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "backward kernel launch failed: %s", hipGetErrorString(e));
  return tsp_host::ok();
}

}  // extern "C"
