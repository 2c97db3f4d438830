// zigzag.h -- the zigzag map from a rank's local query row to its global token position,
// shared by the attention kernels, the device map dump and the host-side helpers.
//
// "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
// Inference", section 2 (Methodology), attention layers: queries are split across ranks
// in a zigzag so that causal attention work is balanced. The sequence is cut into 2*D
// chunks of C tokens; rank r holds chunk r (local rows [0, C)) and chunk 2*D-1-r (local
// rows [C, 2C)). The map is strictly increasing in the local row.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

__host__ __device__ __forceinline__ int32_t tsp_zigzag_position(int32_t row, int32_t C, int32_t D, int32_t rank) {
  return row < C ? rank * C + row : (2 * D - 1 - rank) * C + (row - C);
}
