// Streaming-read probe: reads a buffer once, front to back, with 128-bit
// non-temporal loads. It is the plainest read pattern there is, so its rate
// over a buffer far larger than the caches is the HBM read ceiling of the box
// the other kernels run on; the benchmark reports the decode kernel's KV-read
// rate against it beside the 8.0 TB/s specification. Each workgroup writes
// the wrapping 32-bit sum of the words it read, so no load can be dropped and
// a test can check that every word was read exactly once.

#include "kvc_device.h"
#include "kvc_host.h"

namespace kvc {

constexpr int kProbeGroups = 32768;   // many short workgroups: the fastest grid measured
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;       // 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ data,
                                                                    int64_t n16, uint32_t* out) {
  __shared__ uint32_t wave_sum[kProbeThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  // grid-stride: index i is read by exactly one thread, kProbeUnroll at a time
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(data + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(data + i);
    acc += v.x + v.y + v.z + v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) s += wave_sum[w];
    out[blockIdx.x] = s;
  }
}

}  // namespace kvc

extern "C" int32_t kvc_stream_read_groups(void) { return kvc::kProbeGroups; }

extern "C" int kvc_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream) {
  if (!out || (bytes > 0 && !data)) return KVC_ERR_NULL;
  if (bytes % 16 != 0) return KVC_ERR_SHAPE;
  if (!kvc::aligned_to(data, 16) || !kvc::aligned_to(out, 4)) return KVC_ERR_ALIGN;
  hipLaunchKernelGGL(kvc::stream_read_kernel, dim3(kvc::kProbeGroups), dim3(kvc::kProbeThreads), 0,
                     kvc::as_stream(stream), reinterpret_cast<const kvc::u32x4*>(data),
                     (int64_t)(bytes / 16), out);
  return kvc::launch_status();
}
