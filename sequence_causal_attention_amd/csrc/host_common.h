// host_common.h -- host-side pieces shared by the library's translation units: the
// thread-local error message, argument checks and the query-tile work decomposition.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "attn_common.h"
#include "tsp_attn.h"

namespace tsp_host {

// message of the calling thread's last failed call (defined in tsp_attn.hip)
extern thread_local char g_last_error[512];

inline int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  if (std::getenv("TSP_ATTN_DEBUG")) std::fprintf(stderr, "tsp_attn: %s\n", g_last_error);
  return status;
}

inline int ok() {
  g_last_error[0] = '\0';
  return TSP_OK;
}

inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

inline int check_sizes(int64_t S_total, int64_t D, int64_t rank) {
  if (D < 1) return fail(TSP_EINVAL, "D must be >= 1 (got %lld)", (long long)D);
  if (rank < 0 || rank >= D) return fail(TSP_EINVAL, "rank %lld outside [0, %lld)", (long long)rank, (long long)D);
  if (S_total <= 0) return fail(TSP_EINVAL, "S_total must be > 0 (got %lld)", (long long)S_total);
  if (S_total % (2 * D) != 0)
    return fail(TSP_EINVAL, "S_total %lld not divisible by 2*D = %lld", (long long)S_total, (long long)(2 * D));
  if (S_total > (int64_t(1) << 30)) return fail(TSP_EINVAL, "S_total %lld above 2^30", (long long)S_total);
  return TSP_OK;
}

// Tile configuration of one query-stationary kernel.
struct KernelShape {
  int kv_tile;     // keys per K/V tile
  int waves;       // waves per workgroup
  int row_blocks;  // 32-row query blocks per wave
};

// Validates the sizes (not the pointers, the element type or the head dim) and builds the
// query-tile work decomposition of a query-stationary kernel of shape `ks`.
inline int plan_tiles(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                      const KernelShape& ks, TspParams* p) {
  int st = check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (B < 1) return fail(TSP_EINVAL, "B must be >= 1 (got %lld)", (long long)B);
  if (Hq < 1 || Hkv < 1) return fail(TSP_EINVAL, "Hq and Hkv must be >= 1");
  if (Hq % Hkv != 0) return fail(TSP_EINVAL, "Hq %lld not divisible by Hkv %lld", (long long)Hq, (long long)Hkv);
  if (Hq > 65536 || B > 65536) return fail(TSP_EINVAL, "B or Hq too large");
  // per-lane 32-bit byte offsets span one stage of 64 rows of Hkv*dh (or Hq*dh) elements
  if (Hkv * dh > (int64_t(1) << 22)) return fail(TSP_EINVAL, "Hkv * dh above 2^22");

  const int64_t C = S_total / (2 * D);
  const int64_t grp = Hq / Hkv;
  const int rows_per_wg = 32 * ks.waves * ks.row_blocks;
  // Query heads per workgroup: the largest divisor of grp that also divides the
  // workgroup's row blocks, so one K/V tile in LDS serves as many heads as possible.
  int64_t GH = 1;
  for (int64_t g = 1; g <= grp; ++g)
    if (grp % g == 0 && (ks.waves * ks.row_blocks) % g == 0) GH = g;
  const int64_t BQ = rows_per_wg / GH;
  const int64_t n_qtiles = (2 * C + BQ - 1) / BQ;
  const int64_t n_pairs = (n_qtiles + 1) / 2;
  const int64_t n_units = B * Hkv * (grp / GH) * n_pairs;
  if (n_units > 0x7fffffff) return fail(TSP_EINVAL, "problem too large for one launch");

  p->S_total = (int32_t)S_total;
  p->C = (int32_t)C;
  p->S_local = (int32_t)(2 * C);
  p->D = (int32_t)D;
  p->rank = (int32_t)rank;
  p->Hq = (int32_t)Hq;
  p->Hkv = (int32_t)Hkv;
  p->grp = (int32_t)grp;
  p->GH = (int32_t)GH;
  p->BQ = (int32_t)BQ;
  p->n_qtiles = (int32_t)n_qtiles;
  p->n_pairs = (int32_t)n_pairs;
  p->n_hgroups = (int32_t)(grp / GH);
  p->n_units = (int32_t)n_units;
  p->kv_lo = 0;
  p->kv_hi = (int32_t)S_total;
  p->accumulate = 0;
  p->kv_stride = Hkv * dh;
  p->scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  return TSP_OK;
}

// The attention forward of the library's main unit, for the other units: plan the launch
// (validates sizes, dtype and head dim) and enqueue it.
int attn_plan(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
              TspParams* p);
int attn_launch(const TspParams& p, int64_t dh, int dtype, hipStream_t stream);

// The bf16 forward kernels (tsp_attn_fwd_bf16.hip): the query-tile shape per head dim, and
// the launches of a planned forward (one key range, or two when kv_hi2 > kv_lo2) and of
// the ring sweep over the peers' chunks. Each returns false for a head dim without a
// kernel (nothing is launched then).
bool bf16_kernel_shape(int64_t dh, KernelShape* ks);
bool launch_fwd_bf16(const TspParams& p, int64_t dh, hipStream_t stream);
bool launch_fwd_bf16_ring(const TspParams& p, int64_t dh, hipStream_t stream);

}  // namespace tsp_host
