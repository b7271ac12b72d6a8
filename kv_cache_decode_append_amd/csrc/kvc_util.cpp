// Host-only C-ABI helpers: KV size arithmetic and status strings.
#include "kvc.h"

// 2 (K and V) x layers x kv heads x head dim x bytes per number (aiwithghost.com
// "KV cache and continuous batching: 1,000 people ask AI", section "How KV cache
// memory limits concurrency"; daviddominguez.dev "The KV cache and prefix
// caching", section "What prefill stores and decode reads").
extern "C" int64_t kvc_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                          int32_t dtype_bytes) {
  if (layers < 0 || kv_heads < 0 || head_dim < 0 || dtype_bytes < 0) return -1;
  return (int64_t)2 * layers * kv_heads * head_dim * dtype_bytes;
}

extern "C" const char* kvc_status_string(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_NULL: return "null pointer argument";
    case KVC_ERR_SHAPE: return "inconsistent or negative sizes";
    case KVC_ERR_DTYPE: return "unknown dtype";
    case KVC_ERR_UNSUPPORTED: return "unsupported head_dim, block_size or head grouping";
    case KVC_ERR_WORKSPACE: return "workspace missing or too small";
    case KVC_ERR_LAUNCH: return "kernel launch failed";
    case KVC_ERR_NO_BLOCKS: return "not enough free or reusable blocks";
    case KVC_ERR_STATE: return "block not held, out of range, or cached under another prefix";
    case KVC_ERR_NO_MEMORY: return "host memory ran out";
    case KVC_ERR_ALIGN: return "pointer not aligned as required (16 bytes for tensors and pools)";
    case KVC_ERR_SCRATCH: return "call needs more than the built-in scratch (KVC_SCRATCH_BYTES)";
  }
  return "unknown status";
}
