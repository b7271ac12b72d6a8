// Internal: launcher shared between the append and prefill translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"
#include "kvc_device.h"

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

// Writes 16-byte chunk c of kv head h of row r of a prefill chunk (rows from
// t0 in the packed k/v arrays, positions from p0) into the cache through the
// sequence's block-table row. Returns the error bit for a position the table
// does not cover or a block id outside the pool (nothing is written), else 0.
__device__ __forceinline__ int chunk_append_one(uint8_t* kc, uint8_t* vc, const uint8_t* k,
                                                const uint8_t* v, const int32_t* bt_row,
                                                int32_t max_blocks, int32_t num_blocks,
                                                int32_t hkv, int32_t nc, int32_t t0, int32_t p0,
                                                int32_t r, int32_t h, int32_t c) {
  const int32_t p = p0 + r;
  const int32_t lb = p >> 4;
  if (lb >= max_blocks) return KVC_DEVERR_CONTEXT;
  const int32_t blk = bt_row[lb];
  if (blk < 0 || blk >= num_blocks) return KVC_DEVERR_BLOCK_ID;
  const int64_t row_bytes = (int64_t)nc * 16;
  const int64_t dst = (((int64_t)blk * hkv + h) * 16 + (p & 15)) * row_bytes + (int64_t)c * 16;
  const int64_t src = (((int64_t)(t0 + r) * hkv + h) * nc + c) * 16;
  *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(k + src);
  *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(v + src);
  return 0;
}

}  // namespace kvc
