// attn_common.h -- launch parameters and small device helpers shared by the attention
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zigzag.h"

typedef __bf16 tsp_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 tsp_bf16x2 __attribute__((ext_vector_type(2)));
typedef float tsp_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t tsp_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t tsp_u32x2 __attribute__((ext_vector_type(2)));

// Everything a launch needs; passed by value as the kernel argument.
struct TspParams {
  const void* q;    // [B, S_local, Hq, dh]
  const void* k;    // [B, S_total, Hkv, dh]
  const void* v;    // [B, S_total, Hkv, dh]
  void* out;        // [B, S_local, Hq, dh]
  float* lse;       // [B, Hq, S_local]
  int32_t S_total;  // keys per sequence
  int32_t C;        // chunk length S_total / (2D)
  int32_t S_local;  // 2C local query rows
  int32_t D;        // sequence-parallel degree
  int32_t rank;     // this rank
  int32_t Hq, Hkv, grp;  // query heads, KV heads, Hq / Hkv
  int32_t GH;            // query heads of one KV group handled by one workgroup
  int32_t BQ;            // local rows per query tile
  int32_t n_qtiles;      // ceil(S_local / BQ)
  int32_t n_pairs;       // ceil(n_qtiles / 2): mirrored tile pairs per (b, head group)
  int32_t n_hgroups;     // grp / GH
  int32_t n_units;       // B * Hkv * n_hgroups * n_pairs workgroups
  int32_t kv_lo, kv_hi;  // only keys in [kv_lo, kv_hi) take part (whole sequence: 0, S_total)
  int32_t kv_lo2, kv_hi2;  // and, when kv_hi2 > kv_lo2, the keys in [kv_lo2, kv_hi2) (after kv_hi)
  int32_t accumulate;    // 0: write (out, lse); 1: merge into the (out, lse) already there
  int64_t kv_stride;     // elements between consecutive keys of k / v (Hkv * dh when dense)
  float scale_log2;      // log2(e) / sqrt(dh): scores go straight to the exp2 domain
  // ring sweep (the peers' chunks in arrival order): chunk c may be read once
  // ready[c] == ready_value (ready NULL: every chunk is present); a wait gives up after
  // spin_limit polls and then sets bit 0 of *wait_status
  const int32_t* ready;
  int32_t ready_value;
  int32_t spin_limit;
  int32_t* wait_status;
};


// Workgroup -> work unit. Workgroups are dispatched round-robin over the 8 XCDs
// (block id b lands on XCD b % 8); consecutive units share a KV head, so give each XCD a
// contiguous range of units and the KV tiles they sweep stay in that XCD's L2.
__device__ __forceinline__ int32_t tsp_xcd_unit(int32_t bid, int32_t nblocks) {
  const int32_t xcd = bid & 7;
  const int32_t per = nblocks >> 3, extra = nblocks & 7;
  return xcd * per + (xcd < extra ? xcd : extra) + (bid >> 3);
}

// Max of a value held by lane l and by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float tsp_max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float tsp_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float tsp_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed (low = a).
__device__ __forceinline__ uint32_t tsp_pack_bf16(float a, float b) {
  tsp_bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed pair of bf16 values (one v_dot2 against (1, 1)).
__device__ __forceinline__ float tsp_sum_bf16_pair(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(tsp_bf16x2, packed),
                                         __builtin_bit_cast(tsp_bf16x2, 0x3f803f80u), acc, false);
}

// Units of the lse store: natural log from the base-2 running max and sum.
constexpr float TSP_LN2 = 0.693147180559945309f;

constexpr float TSP_LOG2E = 1.44269504088896340736f;

// Weights of the log-sum-exp merge of a running result (lse_old, natural log, -inf when
// it has no key yet) with a new partial whose lse is m2 + log2(l) in base 2 (l > 0).
// Returns the new natural-log lse; w_old scales the old output, w_new the new partial's
// unnormalised accumulator (1/l folded in).
__device__ __forceinline__ float tsp_merge_weights(float lse_old, float m2, float l, float& w_old,
                                                   float& w_new) {
  const float old2 = lse_old * TSP_LOG2E;  // -inf stays -inf
  const float new2 = m2 + __builtin_amdgcn_logf(l);
  const float m = fmaxf(old2, new2);
  const float e_old = old2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(old2 - m);
  const float e_new = __builtin_amdgcn_exp2f(new2 - m);
  const float tot = e_old + e_new;
  const float inv = 1.0f / tot;
  w_old = e_old * inv;
  w_new = e_new * inv / l;
  return (m + __builtin_amdgcn_logf(tot)) * TSP_LN2;
}

// The running max is only raised when a tile's max exceeds it by more than this many
// base-2 units, so most tiles skip rescaling the accumulators; the unnormalised weights
// stay below 2^TSP_RESCALE_SLACK, far inside fp32 and bf16 range.
constexpr float TSP_RESCALE_SLACK = 8.0f;
