// ulysses_permute.h -- the local layout changes of Ulysses sequence parallelism around
// the one-rank attention ("Tensor, pipeline e sequence parallelism", section 01,
// sequence-parallel paragraph: an all-to-all transposes between sequence partitions and
// head partitions, every rank attends over the whole sequence for a subset of heads, then
// the layout is transposed back; "AutoSP ...", section 2.A items 2-3).
//
// All four changes are one operation on contiguous blocks: a tensor of [M][N] blocks of
// `blk` bytes becomes [N][M] blocks (block (n, m) of the output = block (m, n) of the
// input):
//   pack heads        [B*S_local][P] blocks of (H/P)*dh elements -> [P][B*S_local]
//   unpack heads      [P][B*S_local] -> [B*S_local][P]
//   gather sequence   [P][B] blocks of S_local*(H/P)*dh elements -> [B][P]
//   scatter sequence  [B][P] -> [P][B]
// HBM-bound: every byte is read once and written once. Each thread moves UNROLL 16-byte
// chunks of the output (consecutive threads, consecutive chunks: coalesced stores; the
// loads are contiguous within a block), issuing all its loads before its stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_common.h"

namespace tsp {

struct BlockTransposeParams {
  const tsp_u32x4* in;
  tsp_u32x4* out;
  uint32_t M, N;      // input is [M][N] blocks
  uint32_t cpb;       // 16-byte chunks per block
  uint32_t total;     // M * N * cpb chunks
};

constexpr int TSP_PERMUTE_U = 2;  // output chunks per thread

__global__ __launch_bounds__(256) void block_transpose_kernel(BlockTransposeParams p) {
  constexpr int U = TSP_PERMUTE_U;
  const uint32_t base = blockIdx.x * (256u * U) + threadIdx.x;
  tsp_u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t idx = base + 256u * u;  // output chunk
    if (idx < p.total) {
      const uint32_t ob = idx / p.cpb, c = idx - ob * p.cpb;  // output block (n, m)
      const uint32_t n = ob / p.M, m = ob - n * p.M;
      v[u] = p.in[((uint64_t)m * p.N + n) * p.cpb + c];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t idx = base + 256u * u;
    if (idx < p.total) {
      p.out[idx] = v[u];
    }
  }
}

}  // namespace tsp
