// Paged GQA decode attention with split-K over the context and a merge pass:
// the decode kernel (one 4-wave workgroup per work item, see kvc_decode_item.h
// for the item), the merge kernel and the host entry points.

#include <atomic>

#include "kvc_decode_item.h"
#include "kvc_host.h"

namespace kvc {

constexpr int kWaves = 4;
constexpr int kMaxPartBlocks = kWaves * 64;   // one block id per lane of each wave
constexpr int64_t kMinWorkBlocks = 32;        // blocks a partition should hold when split

template <typename T, int D, int G>
__global__ __launch_bounds__(kWaves * 64) void paged_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeShape<ComputeT<T>, D, G, kWaves>::SMEM];
  // One-dimensional grid, kv head fastest, then sequence, partition slowest:
  // workgroups are dealt round-robin to the 8 XCDs by linear index, so every
  // partition level spreads over all of them. (With the partition fastest, a
  // batch whose sequences mostly need one or two partitions put nearly all
  // the work on one or two XCDs.)
  const int kvh = blockIdx.x % a.hkv;
  const int b = (blockIdx.x / a.hkv) % a.n_seqs;
  const int part = blockIdx.x / (a.n_seqs * a.hkv);
  decode_item<T, D, G, kWaves>(a, kvh, b, part, smem);
}

// One wave per (sequence, query head): combine the partition partials with the
// log-sum-exp rule. Lane j holds partitions j, j + 64, ...: their (m, l) pairs
// are read in one round and the maximum and the normaliser come from wave
// reductions. Each lane then adds the partials of its D/64 output dims in
// partition order, eight partitions' loads in flight at a time, each weight
// read from the lane that holds its partition. The first 64 (m, l) pairs and
// the first eight partitions' partials are read together with the context
// length, before the count of partitions in use is known: the reads stay in
// this row's n_part slots, and what lies past the last used partition (stale
// workspace) is replaced by the neutral value before any arithmetic.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a, int32_t hq_all) {
  const int row = blockIdx.x;                 // b * Hq + hq
  const int b = row / hq_all;
  const int lane = threadIdx.x;
  const float2* ml = a.ws_ml + (size_t)row * a.n_part;
  const float* po = a.ws_o + (size_t)row * a.n_part * D;
  constexpr int E = D >= 64 ? D / 64 : 1;     // output dims per lane
  const bool has = D >= 64 || lane < D;
  const int n_pre = min(8, a.n_part);
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (lane < a.n_part) ml0 = ml[lane];
  float x0[8][E];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) x0[u][e] = (has && u < n_pre) ? po[(size_t)u * D + lane * E + e] : 0.f;
  const int ctx = effective_ctx(a, b, false);
  const int nblk = (ctx + 15) >> 4;
  const int n_used = nblk > 0 ? (nblk + a.part_blocks - 1) / a.part_blocks : 1;
  if (n_used <= 1) return;
  float m_lane = -INFINITY;
  if (lane < n_used) m_lane = fmaxf(m_lane, ml0.x);
  for (int i = lane + 64; i < n_used; i += 64) m_lane = fmaxf(m_lane, ml[i].x);
  const float M = rows_max(group_max<16>(m_lane));
  float l_lane = 0.f;
  if (lane < n_used) l_lane += ml0.y * __builtin_amdgcn_exp2f(ml0.x - M);
  for (int i = lane + 64; i < n_used; i += 64) l_lane += ml[i].y * __builtin_amdgcn_exp2f(ml[i].x - M);
  const float inv = 1.f / rows_sum(group_sum<16>(l_lane));
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int c = 0; c < n_used; c += 64) {      // 64 partitions per round
    float w = 0.f;
    if (c == 0) {
      if (lane < n_used) w = __builtin_amdgcn_exp2f(ml0.x - M);
    } else if (c + lane < n_used) {
      w = __builtin_amdgcn_exp2f(ml[c + lane].x - M);
    }
    const int n = min(64, n_used - c);
    for (int j0 = 0; j0 < n; j0 += 8) {
      float x[8][E];
      if (c == 0 && j0 == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < E; ++e) x[u][e] = u < n ? x0[u][e] : 0.f;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < E; ++e)
            x[u][e] = (has && j0 + u < n) ? po[(size_t)(c + j0 + u) * D + lane * E + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = readlane_f(w, j0 + u);   // 0 past the last partition
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(wu, x[u][e], acc[e]);
      }
    }
  }
  if (has) {
#pragma unroll
    for (int e = 0; e < E; ++e) store_out<ComputeT<T>>(a.out, (size_t)row * D + lane * E + e, acc[e] * inv);
  }
}

template <typename T, int D, int G>
int launch_decode(const DecodeArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL((paged_decode_kernel<T, D, G>), dim3((unsigned)(a.n_part * a.hkv * B)),
                     dim3(kWaves * 64), 0, st, a);
  if (hipGetLastError() != hipSuccess) return KVC_ERR_LAUNCH;
  if (a.n_part > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(B * a.hkv * G), dim3(64), 0, st, a, a.hkv * G);
    if (hipGetLastError() != hipSuccess) return KVC_ERR_LAUNCH;
  }
  return KVC_OK;
}

template <typename T, int D>
int dispatch_g(const DecodeArgs& a, int B, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_decode<T, D, 1>(a, B, st);
    case 2: return launch_decode<T, D, 2>(a, B, st);
    case 4: return launch_decode<T, D, 4>(a, B, st);
    case 8: return launch_decode<T, D, 8>(a, B, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

int dispatch_decode(const DecodeArgs& a, int dtype, int D, int B, int G, hipStream_t st) {
  if (dtype == KVC_F32) {
    switch (D) {
      case 16: return dispatch_g<float, 16>(a, B, G, st);
      case 32: return dispatch_g<float, 32>(a, B, G, st);
      case 64: return dispatch_g<float, 64>(a, B, G, st);
      case 128: return dispatch_g<float, 128>(a, B, G, st);
    }
  } else if (dtype == KVC_BF16) {
    switch (D) {
      case 32: return dispatch_g<bf16_tag, 32>(a, B, G, st);
      case 64: return dispatch_g<bf16_tag, 64>(a, B, G, st);
      case 128: return dispatch_g<bf16_tag, 128>(a, B, G, st);
    }
  } else {
    switch (D) {
      case 64: return dispatch_g<fp8_tag, 64>(a, B, G, st);
      case 128: return dispatch_g<fp8_tag, 128>(a, B, G, st);
    }
  }
  return KVC_ERR_UNSUPPORTED;
}

// Blocks per partition. Every partition costs a pipeline fill, an LDS merge
// and (when a sequence has several) a partial write plus the merge pass, so a
// sequence is split only as far as needed to give the chip about two resident
// workgroups per CU (512 on a 256-CU MI355X). B=64 x 8 kv heads already fills
// that unsplit; 8 sequences at 32k tokens are split 8 ways.
int decode_part_blocks(int B, int hkv, int nblk_max, int cus) {
  const int64_t target = 2 * (int64_t)cus;
  const int64_t units = (int64_t)B * hkv;
  int64_t n_part = (target + units - 1) / units;
  const int64_t max_parts = (nblk_max + kMinPartBlocks - 1) / kMinPartBlocks;
  if (n_part > max_parts) n_part = max_parts;
  if (n_part < 1) n_part = 1;
  // Fewer, longer partitions where a partition would hold few blocks (about 8
  // per wave or fewer): each one's fixed costs (the ring fill, the wave merge,
  // its partial and its share of the merge pass) then outweigh the fuller
  // chip. Halving keeps a power-of-two grid at whole multiples of the CU
  // count (one GPU's share under kv-head x8, 64 rows of ~2k tokens: 4
  // partitions, 4,095 against 3,787 GB/s with 8; 5 or 6 partitions, which
  // give some CUs two workgroups and others one, measured 3,477 and 3,566).
  while (n_part > 1 && (int64_t)nblk_max < kMinWorkBlocks * n_part) n_part = (n_part + 1) / 2;
  int64_t pb = (nblk_max + n_part - 1) / n_part;
  pb = (pb + 3) / 4 * 4;
  if (pb < kMinPartBlocks) pb = kMinPartBlocks;
  if (pb > kMaxPartBlocks) pb = kMaxPartBlocks;
  return (int)pb;
}

}  // namespace kvc

extern "C" size_t kvc_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim,
                                             int32_t max_context_len) {
  if (B <= 0 || Hq <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t nblk = kvc::ceil_div(max_context_len, 16);
  const int64_t n_part_max = kvc::ceil_div(nblk, kvc::kMinPartBlocks);
  if (n_part_max <= 1) return 0;
  return (size_t)B * Hq * n_part_max * ((size_t)head_dim * 4 + 8);
}

namespace kvc {

// Split-K partials of kvc_decode_append_attention_noalloc: one array per
// device, held until the process ends. Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): it uses the
// device address scratch_ptr() returns.
static __device__ __align__(256) uint8_t scratch[KVC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device
// with that device current; nullptr if the runtime cannot give it. Calls from
// several host threads may race to fill an entry, with the same value.
static void* scratch_ptr() {
  static std::atomic<void*> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    cached[dev].store(p, std::memory_order_release);
  }
  return p;
}

// use_scratch: the split-K partials go to `scratch` (workspace ignored), and a
// call needing more than KVC_SCRATCH_BYTES is rejected with KVC_ERR_SCRATCH.
static int decode_entry(const kvc_cache* cache, const void* q, const void* k_new, const void* v_new,
                        int32_t B, int32_t Hq, const int32_t* block_table, int32_t max_blocks,
                        const int32_t* context_lens, int32_t max_context_len, float softmax_scale,
                        void* out, void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch = false) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (B < 0 || Hq <= 0 || max_blocks < 0 || max_context_len < 0) return KVC_ERR_SHAPE;
  if (Hq % cache->num_kv_heads != 0) return KVC_ERR_SHAPE;
  const int G = Hq / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks * 16) return KVC_ERR_SHAPE;
  if (B == 0) return KVC_OK;
  if (!q || !block_table || !context_lens || !out) return KVC_ERR_NULL;

  // the workspace rule is the size query's (it covers the most partitions
  // any device would use), so validation does not depend on the device
  if (use_scratch) workspace = nullptr;
  const size_t ws_rule =
      use_scratch ? 0 : kvc_decode_workspace_bytes(B, Hq, cache->head_dim, max_context_len);
  if (ws_rule > 0 && (!workspace || workspace_bytes < ws_rule)) return KVC_ERR_WORKSPACE;
  if (!cache_aligned(cache) || !all_aligned(16, q, k_new, v_new, out, workspace) ||
      !all_aligned(4, block_table, context_lens))
    return KVC_ERR_ALIGN;

  const int nblk_max = (int)ceil_div(max_context_len, 16);
  const DeviceInfo dev = device_info();
  if (dev.cus == 0) return KVC_ERR_LAUNCH;
  const int pb = decode_part_blocks(B, cache->num_kv_heads, nblk_max, dev.cus);
  const int n_part = nblk_max > 0 ? (int)ceil_div(nblk_max, pb) : 1;
  const size_t n_rows = (size_t)B * Hq * n_part;
  const size_t need = n_part > 1 ? n_rows * ((size_t)cache->head_dim * 4 + 8) : 0;
  if (use_scratch) {
    if (need > KVC_SCRATCH_BYTES) return KVC_ERR_SCRATCH;
    if (need > 0 && (workspace = scratch_ptr()) == nullptr) return KVC_ERR_LAUNCH;
  } else if (need > ws_rule) {
    return KVC_ERR_WORKSPACE;   // cannot happen: pb >= kMinPartBlocks
  }

  DecodeArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kc = cache->k_cache;
  a.vc = cache->v_cache;
  a.bt = block_table;
  a.ctx_lens = context_lens;
  a.out = out;
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_ml = need ? reinterpret_cast<float2*>(reinterpret_cast<uint8_t*>(workspace) +
                                             n_rows * cache->head_dim * 4)
                 : nullptr;
  a.err = cache->err_flag;
  a.hkv = cache->num_kv_heads;
  a.n_seqs = B;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = max_blocks;
  a.max_ctx = max_context_len;
  a.part_blocks = pb;
  a.n_part = n_part;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.ks = cache->k_scale;
  a.vs = cache->v_scale;
  return dispatch_decode(a, cache->dtype, cache->head_dim, B, G, as_stream(stream));
}

}  // namespace kvc

extern "C" int kvc_paged_decode_attention(const kvc_cache* cache, const void* q, int32_t B, int32_t Hq,
                                          const int32_t* block_table, int32_t max_blocks,
                                          const int32_t* context_lens, int32_t max_context_len,
                                          float softmax_scale, void* out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return kvc::decode_entry(cache, q, nullptr, nullptr, B, Hq, block_table, max_blocks, context_lens,
                           max_context_len, softmax_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int kvc_decode_append_attention(const kvc_cache* cache, const void* q, const void* k_new,
                                           const void* v_new, int32_t B, int32_t Hq,
                                           const int32_t* block_table, int32_t max_blocks,
                                           const int32_t* context_lens, int32_t max_context_len,
                                           float softmax_scale, void* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_ERR_NULL;
  return kvc::decode_entry(cache, q, k_new, v_new, B, Hq, block_table, max_blocks, context_lens,
                           max_context_len, softmax_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int kvc_decode_append_attention_noalloc(const kvc_cache* cache, const void* q,
                                                   const void* k_new, const void* v_new, int32_t B,
                                                   int32_t Hq, const int32_t* block_table,
                                                   int32_t max_blocks, const int32_t* context_lens,
                                                   int32_t max_context_len, float softmax_scale,
                                                   void* out, void* stream) {
  if (B > 0 && (!k_new || !v_new)) return KVC_ERR_NULL;
  return kvc::decode_entry(cache, q, k_new, v_new, B, Hq, block_table, max_blocks, context_lens,
                           max_context_len, softmax_scale, out, nullptr, 0, stream, true);
}
