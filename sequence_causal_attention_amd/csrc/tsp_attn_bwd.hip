// tsp_attn_bwd.hip -- C ABI of the backward of the per-rank zigzag / GQA causal attention
// (gfx950): argument validation, work decomposition and dispatch of the three backward
// kernels (attn_bwd_bf16.h); and the allocation-free variant, whose delta lives in a
// static device array of this file.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tsp_attn.h"
#include "attn_bwd_bf16.h"
#include "host_common.h"
#include "bwd_config.h"
#include "attn_bwd_f32.h"

// Workspace of the allocation-free entry point: delta (one float per row and query head)
// in a static device array, one copy per GPU the library runs on, held until the process
// ends. Host code never passes this name to a kernel: on the host it is only a stand-in,
// and its device address comes from hipGetSymbolAddress (see scratch_on_current_device).
constexpr int64_t TSP_BWD_SCRATCH_FLOATS = TSP_BWD_NOALLOC_MAX_ROWS;
static __device__ __align__(256) float scratch[TSP_BWD_SCRATCH_FLOATS];

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

// The device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept; NULL with an error set if the lookup fails.
float* scratch_on_current_device() {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static float* addr[MAX_DEVICES] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    fail(TSP_EINTERNAL, "no current HIP device (or device index above %d)", MAX_DEVICES - 1);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(TSP_EINTERNAL, "hipGetSymbolAddress of the backward workspace failed on device %d: %s", dev,
           hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = static_cast<float*>(ptr);
  }
  return addr[dev];
}

// Pointer checks of the backward's inputs and outputs (delta apart).
int check_bwd_pointers(const void* q_local, const void* k_full, const void* v_full, const void* out,
                       const float* lse, const void* dout, void* dq_local, void* dk_full, void* dv_full) {
  const void* ptrs[] = {q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full};
  for (const void* ptr : ptrs) {
    if (!ptr) return fail(TSP_EINVAL, "null pointer argument");
    if (!aligned16(ptr)) return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  }
  return TSP_OK;
}

// The backward with delta at `delta` (caller's buffer, or the static workspace); pointers
// already checked. `delta_rows_max` > 0 bounds B * Hq * 2C (the workspace's size).
int bwd_impl(const void* q_local, const void* k_full, const void* v_full, const void* out, const float* lse,
             const void* dout, void* dq_local, void* dk_full, void* dv_full, float* delta, int64_t B,
             int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype, void* stream,
             int64_t delta_rows_max) {
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
  if (delta_rows_max > 0 && bp.n_rows > delta_rows_max)
    return fail(TSP_EINVAL, "B * Hq * 2C = %lld rows exceed the static workspace of %lld rows", (long long)bp.n_rows,
                (long long)delta_rows_max);
  if (!delta) {  // the static workspace, only now that the sizes are known to fit
    delta = scratch_on_current_device();
    if (!delta) return TSP_EINTERNAL;
    bp.delta = delta;
  }
  // every buffer the kernels touch must be set by now (a NULL here would reach the kernels
  // as a wild address)
  const void* launch_ptrs[] = {bp.f.q, bp.f.k, bp.f.v, bp.f.out, bp.f.lse, bp.dout, bp.dq, bp.dk, bp.dv, bp.delta};
  for (const void* ptr : launch_ptrs)
    if (!ptr) return fail(TSP_EINTERNAL, "backward launch with an unset buffer pointer");
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

}  // namespace

extern "C" {

int tsp_attn_bwd(const void* q_local, const void* k_full, const void* v_full, const void* out, const float* lse,
                 const void* dout, void* dq_local, void* dk_full, void* dv_full, float* delta, int64_t B,
                 int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
                 void* stream) {
  int st = check_bwd_pointers(q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full);
  if (st != TSP_OK) return st;
  if (!delta) return fail(TSP_EINVAL, "null pointer argument");
  if (!aligned16(delta)) return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  return bwd_impl(q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full, delta, B, S_total, D, rank, Hq,
                  Hkv, dh, dtype, stream, 0);
}

int tsp_attn_bwd_noalloc(const void* q_local, const void* k_full, const void* v_full, const void* out,
                         const float* lse, const void* dout, void* dq_local, void* dk_full, void* dv_full, int64_t B,
                         int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
                         void* stream) {
  int st = check_bwd_pointers(q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full);
  if (st != TSP_OK) return st;
  return bwd_impl(q_local, k_full, v_full, out, lse, dout, dq_local, dk_full, dv_full, nullptr, B, S_total, D, rank,
                  Hq, Hkv, dh, dtype, stream, TSP_BWD_SCRATCH_FLOATS);
}

}  // extern "C"
