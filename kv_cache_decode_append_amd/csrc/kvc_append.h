// Internal: launcher shared between the append and prefill translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// Writes each sequence's prefill chunk K/V at positions prefix .. prefix + C - 1.
int launch_chunk_append(const kvc_cache* c, const void* k, const void* v, int32_t n_seqs,
                        const int32_t* cu, const int32_t* prefix, int32_t total, int32_t max_chunk,
                        const int32_t* block_table, int32_t max_blocks, hipStream_t st);

// A chunk descriptor the kernels may trust: rows t0 .. t0+C-1 lie inside the
// packed arrays, the chunk fits the grid and the prefix is not negative.
__device__ __forceinline__ bool chunk_ok(int t0, int C, int p0, int total, int max_chunk) {
  return t0 >= 0 && C >= 0 && C <= max_chunk && t0 + C <= total && p0 >= 0;
}

}  // namespace kvc
