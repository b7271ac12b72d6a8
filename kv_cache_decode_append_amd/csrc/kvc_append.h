// Internal: launcher shared between the append and prefill translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// Writes each sequence's prefill chunk K/V at positions prefix .. prefix + C - 1.
int launch_chunk_append(const kvc_cache* c, const void* k, const void* v, int32_t n_seqs,
                        const int32_t* cu, const int32_t* prefix, int32_t max_chunk,
                        const int32_t* block_table, int32_t max_blocks, hipStream_t st);

}  // namespace kvc
