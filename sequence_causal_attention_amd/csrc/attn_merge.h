// attn_merge.h -- combine two partial attention results over disjoint key sets.
//
// With the K/V all-gather overlapped with computation ("Folding Tensor and Sequence
// Parallelism ...", section 2, attention layers, and section 3 item 3), a rank attends to
// each gathered chunk of keys as it arrives; the partial results (out_x, lse_x) are
// combined with the log-sum-exp rule:
//   lse = log(exp(lse_a) + exp(lse_b)),  out = exp(lse_a - lse) out_a + exp(lse_b - lse) out_b,
// where a partial with lse = -inf (no visible key) contributes nothing.
//
// HBM-bound elementwise kernel: each thread owns 16 bytes of one output row
// (b, i, h): it reads that row's two lse values and 16 bytes of each partial, and
// writes 16 bytes; the thread holding the row's first chunk writes the merged lse.
// All threads of a row are in one wave, so out / lse may alias out_a / lse_a (the wave
// reads every input before any lane stores).
#pragma once

#include "attn_common.h"

namespace tsp {

struct MergeParams {
  const void* out_a;
  const float* lse_a;
  const void* out_b;
  const float* lse_b;
  void* out;
  float* lse;
  int64_t rows;      // B * S_local * Hq
  int32_t S_local;   // local rows per (b, h)
  int32_t Hq;
};

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int EPT = 16 / sizeof(T);  // elements per thread (16 bytes)
  constexpr int TPR = DH / EPT;        // threads per row
  static_assert(64 % TPR == 0, "a row must not straddle two waves");
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = tid / TPR;
  if (row >= p.rows) return;
  const int c = (int)(tid % TPR);
  // row = ((b * S_local) + i) * Hq + h  ->  lse index (b * Hq + h) * S_local + i
  const int32_t h = (int32_t)(row % p.Hq);
  const int64_t bi = row / p.Hq;
  const int32_t i = (int32_t)(bi % p.S_local);
  const int64_t b = bi / p.S_local;
  const int64_t li = (b * p.Hq + h) * p.S_local + i;
  const float la = p.lse_a[li], lb = p.lse_b[li];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float ea = la == -INFINITY ? 0.f : __expf(la - m);
    const float eb = lb == -INFINITY ? 0.f : __expf(lb - m);
    const float tot = ea + eb;
    wa = ea / tot;
    wb = eb / tot;
    lse = m + __logf(tot);
  }
  const int64_t off = row * DH + (int64_t)c * EPT;
  const tsp_u32x4 xa = *reinterpret_cast<const tsp_u32x4*>(static_cast<const T*>(p.out_a) + off);
  const tsp_u32x4 xb = *reinterpret_cast<const tsp_u32x4*>(static_cast<const T*>(p.out_b) + off);
  tsp_u32x4 y;
  if constexpr (sizeof(T) == 2) {  // bf16: unpack pairs, blend in fp32, round to nearest even
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a0 = __uint_as_float(xa[w] << 16), a1 = __uint_as_float(xa[w] & 0xffff0000u);
      const float b0 = __uint_as_float(xb[w] << 16), b1 = __uint_as_float(xb[w] & 0xffff0000u);
      y[w] = tsp_pack_bf16(fmaf(wa, a0, wb * b0), fmaf(wa, a1, wb * b1));
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      y[w] = __float_as_uint(fmaf(wa, __uint_as_float(xa[w]), wb * __uint_as_float(xb[w])));
  }
  *reinterpret_cast<tsp_u32x4*>(static_cast<T*>(p.out) + off) = y;
  if (c == 0) p.lse[li] = lse;
}

}  // namespace tsp
