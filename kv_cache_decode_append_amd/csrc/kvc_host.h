// Host-side helpers shared by the kvc C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kvc.h"

namespace kvc {

// Bytes of one cached element (codes only for KVC_FP8).
inline int dtype_bytes(int32_t dtype) {
  return dtype == KVC_F32 ? 4 : dtype == KVC_BF16 ? 2 : dtype == KVC_FP8 ? 1 : 0;
}

inline bool head_dim_supported(int32_t dtype, int32_t d) {
  if (dtype == KVC_F32) return d == 16 || d == 32 || d == 64 || d == 128;
  if (dtype == KVC_BF16) return d == 32 || d == 64 || d == 128;
  if (dtype == KVC_FP8) return d == 64 || d == 128;
  return false;
}

// Validates a cache descriptor; returns KVC_OK or a negative status.
inline int check_cache(const kvc_cache* c) {
  if (!c || !c->k_cache || !c->v_cache) return KVC_ERR_NULL;
  if (dtype_bytes(c->dtype) == 0) return KVC_ERR_DTYPE;
  if (c->dtype == KVC_FP8 && (!c->k_scale || !c->v_scale)) return KVC_ERR_NULL;
  if (c->block_size != 16) return KVC_ERR_UNSUPPORTED;
  if (c->num_blocks < 0 || c->num_kv_heads <= 0) return KVC_ERR_SHAPE;
  if (!head_dim_supported(c->dtype, c->head_dim)) return KVC_ERR_UNSUPPORTED;
  // 32-bit slot numbers and per-tile byte offsets
  if ((int64_t)c->num_blocks * c->block_size > INT32_MAX) return KVC_ERR_SHAPE;
  return KVC_OK;
}

// Alignment the kernels rely on: 16 bytes for what they move in 16-byte
// chunks (q, k, v, out, the K / V pools, workspaces), 4 for int32 arrays and
// the fp8 scale pools, 8 for int64 slot lists. NULL passes (an optional
// pointer, or one already rejected).
inline bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}
template <class... P>
inline bool all_aligned(uintptr_t a, P... p) {
  return (aligned_to(p, a) && ...);
}
inline bool cache_aligned(const kvc_cache* c) {
  return all_aligned(16, c->k_cache, c->v_cache) && all_aligned(4, c->k_scale, c->v_scale, c->err_flag);
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units and XCDs (accelerator complex dies, each with its own L2) of
// the current device, queried once per device and cached; {0, 0} if the
// runtime cannot say. Calls from several host threads may race to fill an
// entry, with the same values.
struct DeviceInfo {
  int cus;
  int xcds;
};
inline DeviceInfo device_info() {
  static std::atomic<int> cached_cus[64], cached_xcds[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return {0, 0};
  int cus = cached_cus[dev].load(std::memory_order_relaxed);
  int xcds = cached_xcds[dev].load(std::memory_order_relaxed);
  if (cus == 0 || xcds == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
        cus <= 0 || xcds <= 0)
      return {0, 0};
    cached_cus[dev].store(cus, std::memory_order_relaxed);
    cached_xcds[dev].store(xcds, std::memory_order_relaxed);
  }
  return {cus, xcds};
}

}  // namespace kvc
