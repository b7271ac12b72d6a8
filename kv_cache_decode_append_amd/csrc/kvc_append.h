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

// fp8 cache: the 8 values of chunk c of kv head h of row r (packed bf16 k/v,
// rows from t0, positions from p0, as chunk_append_one), coded with their
// row's scale: amax / 448 over the row, codes = E4M3(x * 448 / amax), a row
// below kZeroRowAmax stored as zeros with scale 0. The NCB = head_dim / 8
// lanes of one row must form an aligned group of 8 or 16 lanes and all call
// this together (the amax is a reduction over the group); a lane whose `in`
// is false only takes part in the reduction. Returns the error bit as
// chunk_append_one does (nothing written for that row).
template <int NCB>
__device__ __forceinline__ int chunk_append_fp8_one(uint8_t* kc, uint8_t* vc, float* ks, float* vs,
                                                    const uint8_t* k, const uint8_t* v,
                                                    const int32_t* bt_row, int32_t max_blocks,
                                                    int32_t num_blocks, int32_t hkv, int32_t t0,
                                                    int32_t p0, int32_t r, int32_t h, int32_t c,
                                                    bool in) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int64_t src = (((int64_t)(t0 + r) * hkv + h) * NCB + c) * 16;
  const u32x4 kx = in ? *reinterpret_cast<const u32x4*>(k + src) : zero;
  const u32x4 vx = in ? *reinterpret_cast<const u32x4*>(v + src) : zero;
  const float ka = group_max<NCB>(bf16x8_amax(kx));
  const float va = group_max<NCB>(bf16x8_amax(vx));
  if (!in) return 0;
  const int32_t p = p0 + r, lb = p >> 4;
  if (lb >= max_blocks) return KVC_DEVERR_CONTEXT;
  const int32_t blk = bt_row[lb];
  if (blk < 0 || blk >= num_blocks) return KVC_DEVERR_BLOCK_ID;
  const int64_t prow = ((int64_t)blk * hkv + h) * 16 + (p & 15);
  const bool kz = !(ka >= kZeroRowAmax), vz = !(va >= kZeroRowAmax);
  *reinterpret_cast<u32x2*>(kc + prow * (NCB * 8) + c * 8) =
      kz ? u32x2{0u, 0u} : bf16x8_to_e4m3x8(kx, kE4M3Max / ka);
  *reinterpret_cast<u32x2*>(vc + prow * (NCB * 8) + c * 8) =
      vz ? u32x2{0u, 0u} : bf16x8_to_e4m3x8(vx, kE4M3Max / va);
  if (c == 0) {
    ks[prow] = kz ? 0.f : ka / kE4M3Max;
    vs[prow] = vz ? 0.f : va / kE4M3Max;
  }
  return 0;
}

}  // namespace kvc
