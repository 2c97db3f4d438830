// tsp_attn.hip -- C ABI of the per-rank zigzag / GQA causal attention forward (gfx950):
// argument validation, work decomposition, kernel dispatch, the fp32 forward, the merge,
// the Ulysses layout changes, the zigzag map helpers and the error strings. The bf16
// forward kernels live in tsp_attn_fwd_bf16.hip (their own code-generation flags). The
// operation and every argument are documented in tsp_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tsp_attn.h"
#include "attn_common.h"
#include "attn_fwd_f32.h"
#include "attn_merge.h"
#include "ulysses_permute.h"
#include "host_common.h"

namespace tsp_host {
thread_local char g_last_error[512] = "";
}

namespace {

using tsp_host::aligned16;
using tsp_host::check_sizes;
using tsp_host::fail;
using tsp_host::KernelShape;

bool kernel_shape(int dtype, int64_t dh, KernelShape* ks) {
  if (dtype == TSP_BF16) return tsp_host::bf16_kernel_shape(dh, ks);
  if (dtype == TSP_F32 && (dh == 64 || dh == 128 || dh == 256)) {
    *ks = KernelShape{32, 4, 1};
    return true;
  }
  return false;
}

// Validates everything but pointers and builds the launch parameters.
int plan(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
         TspParams* p, KernelShape* ks) {
  int st = check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (dtype != TSP_BF16 && dtype != TSP_F32) return fail(TSP_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (!kernel_shape(dtype, dh, ks)) return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
  return tsp_host::plan_tiles(B, S_total, D, rank, Hq, Hkv, dh, *ks, p);
}

template <int DH>
void launch_f32(const TspParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((tsp::attn_fwd_f32_kernel<DH>), dim3(p.n_units), dim3(256), 0, stream, p);
}

// Validates a Ulysses layout change and launches the block transpose of [M][N] blocks.
int ulysses_transpose(const char* what, const void* in, void* out, int64_t B, int64_t S_local, int64_t H,
                      int64_t dh, int64_t P, int dtype, bool heads, bool forward, void* stream) {
  if (!in || !out) return fail(TSP_EINVAL, "%s: null pointer argument", what);
  if (!aligned16(in) || !aligned16(out)) return fail(TSP_EINVAL, "%s: pointers must be 16-byte aligned", what);
  if (B < 1 || S_local < 1 || H < 1 || dh < 1 || P < 1)
    return fail(TSP_EINVAL, "%s: B, S_local, heads, dh and P must be >= 1", what);
  if (dtype != TSP_BF16 && dtype != TSP_F32) return fail(TSP_EUNSUPPORTED, "%s: unknown dtype %d", what, dtype);
  const int64_t eb = dtype == TSP_BF16 ? 2 : 4;
  if ((dh * eb) % 16 != 0) return fail(TSP_EUNSUPPORTED, "%s: dh * element size must be a multiple of 16", what);
  if (heads && H % P != 0) return fail(TSP_EINVAL, "%s: H %lld not divisible by P %lld", what, (long long)H, (long long)P);
  // heads: H is the total head count; sequence: H is the heads per rank
  const int64_t hl = heads ? H / P : H;
  const int64_t blk = heads ? hl * dh * eb : S_local * hl * dh * eb;
  const int64_t outer = heads ? B * S_local : B;  // the index that stays with the tokens
  const int64_t total = outer * P * (blk / 16);
  if (total >= (int64_t(1) << 32)) return fail(TSP_EINVAL, "%s: tensor above 64 GiB", what);
  tsp::BlockTransposeParams bp{};
  bp.in = static_cast<const tsp_u32x4*>(in);
  bp.out = static_cast<tsp_u32x4*>(out);
  // pack heads / scatter sequence: [outer][P] -> [P][outer]; the inverses: [P][outer] -> [outer][P]
  const bool to_rank_major = heads ? forward : !forward;
  bp.M = (uint32_t)(to_rank_major ? outer : P);
  bp.N = (uint32_t)(to_rank_major ? P : outer);
  bp.cpb = (uint32_t)(blk / 16);
  bp.total = (uint32_t)total;
  const int64_t per_wg = 256 * tsp::TSP_PERMUTE_U;
  (void)hipGetLastError();
  hipLaunchKernelGGL(tsp::block_transpose_kernel, dim3((unsigned)((total + per_wg - 1) / per_wg)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return tsp_host::ok();
}

__global__ void zigzag_dump_kernel(int32_t* out, int32_t n, int32_t C, int32_t D, int32_t rank) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = tsp_zigzag_position(i, C, D, rank);
}

}  // namespace

namespace tsp_host {

int attn_plan(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
              TspParams* p) {
  KernelShape ks{};
  return plan(B, S_total, D, rank, Hq, Hkv, dh, dtype, p, &ks);
}

int attn_launch(const TspParams& p, int64_t dh, int dtype, hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype == TSP_BF16) {
    if (!tsp_host::launch_fwd_bf16(p, dh, stream))
      return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
  } else {
    switch (dh) {
      case 64: launch_f32<64>(p, stream); break;
      case 128: launch_f32<128>(p, stream); break;
      case 256: launch_f32<256>(p, stream); break;
      default: return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "attention kernel launch failed: %s", hipGetErrorString(e));
  return TSP_OK;
}

}  // namespace tsp_host

extern "C" {

int tsp_attn_fwd_range2(const void* q_local, const void* k_full, const void* v_full, void* out, float* lse,
                        int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                        int64_t kv_begin, int64_t kv_end, int64_t kv_begin2, int64_t kv_end2, int accumulate,
                        int dtype, void* stream) {
  if (!q_local || !k_full || !v_full || !out || !lse) return fail(TSP_EINVAL, "null pointer argument");
  if (!aligned16(q_local) || !aligned16(k_full) || !aligned16(v_full) || !aligned16(out) || !aligned16(lse))
    return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  TspParams p{};
  KernelShape ks{};
  int st = plan(B, S_total, D, rank, Hq, Hkv, dh, dtype, &p, &ks);
  if (st != TSP_OK) return st;
  if (kv_begin < 0 || kv_begin > kv_end || kv_end > S_total)
    return fail(TSP_EINVAL, "key range [%lld, %lld) not inside [0, %lld]", (long long)kv_begin,
                (long long)kv_end, (long long)S_total);
  if (kv_begin2 > kv_end2 || kv_end2 > S_total || (kv_end2 > kv_begin2 && kv_begin2 < kv_end))
    return fail(TSP_EINVAL, "second key range [%lld, %lld) must lie inside [%lld, %lld]", (long long)kv_begin2,
                (long long)kv_end2, (long long)kv_end, (long long)S_total);
  if (accumulate != 0 && accumulate != 1) return fail(TSP_EINVAL, "accumulate must be 0 or 1");
  // Keys past the rank's last query position (the end of its second chunk) are visible to
  // no row: clip both ranges there, then let one range stand for two where the other is
  // empty or they touch. The visible keys are the same; a single range runs the one-range
  // kernel and, for fp32, one launch.
  const int64_t seen = (2 * D - rank) * (S_total / (2 * D));  // keys [0, seen) are visible to some row
  int64_t lo1 = kv_begin, hi1 = std::max(kv_begin, std::min(kv_end, seen));
  int64_t lo2 = kv_begin2, hi2 = std::max(kv_begin2, std::min(kv_end2, seen));
  if (hi1 == lo1) {  // the first range is empty: the second alone (or nothing)
    lo1 = lo2;
    hi1 = hi2;
    lo2 = hi2 = S_total;
  } else if (hi2 > lo2 && lo2 == hi1) {  // adjacent ranges: one range
    hi1 = hi2;
    lo2 = hi2 = S_total;
  }
  const bool two = hi2 > lo2;
  p.kv_lo = (int32_t)lo1;
  p.kv_hi = (int32_t)hi1;
  p.accumulate = accumulate;
  p.q = q_local;
  p.k = k_full;
  p.v = v_full;
  p.out = out;
  p.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below reports this launch
  if (dtype == TSP_BF16) {
    if (two) {  // one sweep over both ranges
      p.kv_lo2 = (int32_t)lo2;
      p.kv_hi2 = (int32_t)hi2;
    }
    tsp_host::launch_fwd_bf16(p, dh, s);
  } else {
    // fp32: one launch per range, the second merged into the first's result
    for (int rg = 0; rg < (two ? 2 : 1); ++rg) {
      if (rg == 1) {
        p.kv_lo = (int32_t)lo2;
        p.kv_hi = (int32_t)hi2;
        p.accumulate = 1;
      }
      switch (dh) {
        case 64: launch_f32<64>(p, s); break;
        case 128: launch_f32<128>(p, s); break;
        case 256: launch_f32<256>(p, s); break;
      }
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return tsp_host::ok();
}

int tsp_attn_fwd_range(const void* q_local, const void* k_full, const void* v_full, void* out, float* lse,
                       int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                       int64_t kv_begin, int64_t kv_end, int accumulate, int dtype, void* stream) {
  return tsp_attn_fwd_range2(q_local, k_full, v_full, out, lse, B, S_total, D, rank, Hq, Hkv, dh, kv_begin, kv_end,
                             S_total, S_total, accumulate, dtype, stream);
}

int tsp_attn_fwd_ring(const void* q_local, const void* k_full, const void* v_full, void* out, float* lse,
                      int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                      const int32_t* chunk_ready, int32_t ready_value, int32_t spin_limit, int32_t* wait_status,
                      int dtype, void* stream) {
  if (!q_local || !k_full || !v_full || !out || !lse) return fail(TSP_EINVAL, "null pointer argument");
  if (!aligned16(q_local) || !aligned16(k_full) || !aligned16(v_full) || !aligned16(out) || !aligned16(lse))
    return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  if (chunk_ready && (!wait_status || spin_limit < 1))
    return fail(TSP_EINVAL, "with arrival flags, wait_status must be given and spin_limit must be >= 1");
  TspParams p{};
  KernelShape ks{};
  int st = plan(B, S_total, D, rank, Hq, Hkv, dh, dtype, &p, &ks);
  if (st != TSP_OK) return st;
  if (dtype != TSP_BF16) return fail(TSP_EUNSUPPORTED, "the ring sweep has a bf16 kernel only");
  // every query tile lies in one chunk, and every chunk is whole stages (64 keys)
  if (p.C % p.BQ != 0 || p.C % 64 != 0)
    return fail(TSP_EUNSUPPORTED, "the ring sweep needs the chunk length (%d) to be a multiple of the query tile (%d) "
                "and of 64", p.C, p.BQ);
  // the rank's own two chunks first: one two-range launch, written fresh
  const int64_t C = S_total / (2 * D);
  st = tsp_attn_fwd_range2(q_local, k_full, v_full, out, lse, B, S_total, D, rank, Hq, Hkv, dh, rank * C,
                           (rank + 1) * C, (2 * D - 1 - rank) * C, (2 * D - rank) * C, 0, dtype, stream);
  if (st != TSP_OK || D == 1) return st;
  // then the peers' chunks in arrival order, merged into that result in the epilogue
  p.q = q_local;
  p.k = k_full;
  p.v = v_full;
  p.out = out;
  p.lse = lse;
  p.accumulate = 1;
  p.ready = chunk_ready;
  p.ready_value = ready_value;
  p.spin_limit = spin_limit;
  p.wait_status = wait_status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  tsp_host::launch_fwd_bf16_ring(p, dh, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return tsp_host::ok();
}

int tsp_attn_fwd(const void* q_local, const void* k_full, const void* v_full, void* out, float* lse, int64_t B,
                 int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh, int dtype,
                 void* stream) {
  return tsp_attn_fwd_range(q_local, k_full, v_full, out, lse, B, S_total, D, rank, Hq, Hkv, dh, 0, S_total, 0,
                            dtype, stream);
}

int tsp_attn_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b, void* out,
                   float* lse, int64_t B, int64_t S_local, int64_t Hq, int64_t dh, int dtype, void* stream) {
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return fail(TSP_EINVAL, "null pointer argument");
  if (!aligned16(out_a) || !aligned16(out_b) || !aligned16(out) || !aligned16(lse_a) || !aligned16(lse_b) ||
      !aligned16(lse))
    return fail(TSP_EINVAL, "pointers must be 16-byte aligned");
  if (B < 1 || S_local < 1 || Hq < 1) return fail(TSP_EINVAL, "B, S_local and Hq must be >= 1");
  if (S_local > 0x7fffffff || Hq > 65536 || B > 65536) return fail(TSP_EINVAL, "sizes too large");
  if (dtype != TSP_BF16 && dtype != TSP_F32) return fail(TSP_EUNSUPPORTED, "unknown dtype %d", dtype);
  if (dh != 64 && dh != 128 && dh != 256) return fail(TSP_EUNSUPPORTED, "head dim %lld not in {64, 128, 256}", (long long)dh);
  tsp::MergeParams mp{out_a, lse_a, out_b, lse_b, out, lse, B * S_local * Hq, (int32_t)S_local, (int32_t)Hq};
  const int ept = dtype == TSP_BF16 ? 8 : 4;
  const int64_t threads = mp.rows * (dh / ept);
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == TSP_BF16) {
    switch (dh) {
      case 64: hipLaunchKernelGGL((tsp::attn_merge_kernel<uint16_t, 64>), grid, dim3(256), 0, st, mp); break;
      case 128: hipLaunchKernelGGL((tsp::attn_merge_kernel<uint16_t, 128>), grid, dim3(256), 0, st, mp); break;
      case 256: hipLaunchKernelGGL((tsp::attn_merge_kernel<uint16_t, 256>), grid, dim3(256), 0, st, mp); break;
    }
  } else {
    switch (dh) {
      case 64: hipLaunchKernelGGL((tsp::attn_merge_kernel<float, 64>), grid, dim3(256), 0, st, mp); break;
      case 128: hipLaunchKernelGGL((tsp::attn_merge_kernel<float, 128>), grid, dim3(256), 0, st, mp); break;
      case 256: hipLaunchKernelGGL((tsp::attn_merge_kernel<float, 256>), grid, dim3(256), 0, st, mp); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "merge kernel launch failed: %s", hipGetErrorString(e));
  return tsp_host::ok();
}

int tsp_ulysses_pack_heads(const void* x, void* send, int64_t B, int64_t S_local, int64_t H, int64_t dh, int64_t P,
                           int dtype, void* stream) {
  return ulysses_transpose("pack_heads", x, send, B, S_local, H, dh, P, dtype, true, true, stream);
}

int tsp_ulysses_unpack_heads(const void* send, void* x, int64_t B, int64_t S_local, int64_t H, int64_t dh,
                             int64_t P, int dtype, void* stream) {
  return ulysses_transpose("unpack_heads", send, x, B, S_local, H, dh, P, dtype, true, false, stream);
}

int tsp_ulysses_gather_sequence(const void* recv, void* full, int64_t B, int64_t S_local, int64_t Hl, int64_t dh,
                                int64_t P, int dtype, void* stream) {
  return ulysses_transpose("gather_sequence", recv, full, B, S_local, Hl, dh, P, dtype, false, true, stream);
}

int tsp_ulysses_scatter_sequence(const void* full, void* send, int64_t B, int64_t S_local, int64_t Hl, int64_t dh,
                                 int64_t P, int dtype, void* stream) {
  return ulysses_transpose("scatter_sequence", full, send, B, S_local, Hl, dh, P, dtype, false, false, stream);
}

int tsp_attn_zigzag_positions(int64_t S_total, int64_t D, int64_t rank, int64_t* out_host) {
  int st = check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (!out_host) return fail(TSP_EINVAL, "null output pointer");
  const int32_t C = (int32_t)(S_total / (2 * D));
  for (int32_t i = 0; i < 2 * C; ++i) out_host[i] = tsp_zigzag_position(i, C, (int32_t)D, (int32_t)rank);
  return TSP_OK;
}

int tsp_attn_zigzag_positions_device(int32_t* out_dev, int64_t S_total, int64_t D, int64_t rank, void* stream) {
  int st = check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  if (!out_dev) return fail(TSP_EINVAL, "null output pointer");
  const int32_t C = (int32_t)(S_total / (2 * D));
  const int32_t n = 2 * C;
  (void)hipGetLastError();
  hipLaunchKernelGGL(zigzag_dump_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                     out_dev, n, C, (int32_t)D, (int32_t)rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TSP_ELAUNCH, "map kernel launch failed: %s", hipGetErrorString(e));
  return TSP_OK;
}

int64_t tsp_attn_unmasked_pairs(int64_t S_total, int64_t D, int64_t rank) {
  int st = check_sizes(S_total, D, rank);
  if (st != TSP_OK) return st;
  const int32_t C = (int32_t)(S_total / (2 * D));
  int64_t total = 0;
  for (int32_t i = 0; i < 2 * C; ++i) total += (int64_t)tsp_zigzag_position(i, C, (int32_t)D, (int32_t)rank) + 1;
  return total;
}

int tsp_attn_schedule(int64_t B, int64_t S_total, int64_t D, int64_t rank, int64_t Hq, int64_t Hkv, int64_t dh,
                      int dtype, int64_t* n_workgroups, int64_t* kv_tiles_per_workgroup, int64_t* kv_tile) {
  if (!n_workgroups) return fail(TSP_EINVAL, "null n_workgroups");
  TspParams p{};
  KernelShape ks{};
  int st = plan(B, S_total, D, rank, Hq, Hkv, dh, dtype, &p, &ks);
  if (st != TSP_OK) return st;
  *n_workgroups = p.n_units;
  if (kv_tile) *kv_tile = ks.kv_tile;
  if (kv_tiles_per_workgroup) {
    for (int64_t u = 0; u < p.n_units; ++u) {
      const int32_t pair = (int32_t)(u % p.n_pairs);
      int64_t tiles = 0;
      for (int which = 0; which < 2; ++which) {
        const int32_t qt = which == 0 ? p.n_qtiles - 1 - pair : pair;
        if (which == 1 && qt == p.n_qtiles - 1 - pair) break;
        const int32_t last_row = std::min(qt * p.BQ + p.BQ, p.S_local) - 1;
        const int64_t kv_end = (int64_t)tsp_zigzag_position(last_row, p.C, p.D, p.rank) + 1;
        tiles += (kv_end + ks.kv_tile - 1) / ks.kv_tile;
      }
      kv_tiles_per_workgroup[u] = tiles;
    }
  }
  return TSP_OK;
}

const char* tsp_attn_strerror(int status) {
  switch (status) {
    case TSP_OK: return "success";
    case TSP_EINVAL: return "invalid argument";
    case TSP_EUNSUPPORTED: return "unsupported head dimension or element type";
    case TSP_ELAUNCH: return "kernel launch failed";
    case TSP_EINTERNAL: return "internal HIP runtime error";
    default: return "unknown status";
  }
}

const char* tsp_attn_last_error(void) { return tsp_host::g_last_error; }

}  // extern "C"
