// Chunked-prefill attention: write a prompt chunk's K/V into the paged cache,
// then causal attention of every chunk position over the cached prefix and the
// chunk's own positions up to itself (the work item is in kvc_prefill_item.h),
// with optional key-range splits and their merge kernel, and the host entry
// points.

#include <algorithm>

#include "kvc_host.h"
#include "kvc_prefill_item.h"

namespace kvc {

// Work item of this workgroup. Workgroups are dealt round-robin to the XCDs
// (8 on MI355X), and each XCD runs the items it is given in order. A group
// (the query tiles of one sequence and kv head) stays on one XCD, so its tiles
// share that L2 while they sweep the same keys. Handing each XCD a contiguous
// run of groups would, for a few sequences of different lengths, leave the
// XCDs that drew the long ones working alone at the end; so (when there are
// more items than CUs, the groups fill the XCDs evenly and there are at most
// 64 sequences) the groups are ranked by cost, chunk length x mean keys per
// query, and dealt to the XCDs in snake order, costliest first: every XCD gets
// an even share and starts with its largest.
__device__ __forceinline__ int prefill_work(const PrefillArgs& a) {
  const int nx = a.n_xcd;
  const int x = blockIdx.x % nx, j = blockIdx.x / nx;
  const int per_xcd = gridDim.x / nx;
  const int ipg = a.n_qt * a.n_split;                 // items per group: qt fastest, then split
  const int n_groups = a.n_work / ipg;
  const int n_seqs = n_groups / a.hkv;
  // with no more items than CUs every workgroup has a CU of its own and the
  // order does not matter; the ranking would only add a read before the start
  if (a.n_work <= a.n_cus || n_groups % nx != 0 || n_seqs > kMaxRankedSeqs || per_xcd * nx != a.n_work)
    return x * per_xcd + j;
  const int k = j / ipg, t = j % ipg;
  const int r = nx * k + ((k & 1) ? nx - 1 - x : x);  // rank of the group, 0 = costliest
  const int s = seq_with_cost_rank(a, n_seqs, r / a.hkv), kvh = r % a.hkv;
  return t + ipg * (kvh + a.hkv * s);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kPfThreads) void prefill_attention_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PfShape<PfComputeT<T>, D, G>::SMEM];
  const int work = prefill_work(a);
  if (work >= a.n_work) return;
  prefill_item<T, D, G>(a, work, smem);
}

// One wave per (token, query head): combine the key-range partials of a split
// prefill with the log-sum-exp rule (the same rule the split decode uses).
// Lane j holds ranges j, j + 64, ...: their (m, l) pairs are read in one round,
// the maximum and the normaliser come from wave reductions, and each lane adds
// the partials of its D/64 output dims in range order, eight ranges' loads in
// flight at a time. A range holding no key of the row (m = -inf) adds nothing.
template <typename T, int D>
__global__ __launch_bounds__(64) void prefill_merge_kernel(PrefillArgs a, int32_t hq_all) {
  const size_t row = blockIdx.x;                       // token * Hq + head
  if (row >= (size_t)a.total * hq_all) return;
  const int lane = threadIdx.x, n_split = a.n_split;
  const float2* ml = a.ws_ml + row * n_split;
  const float* po = a.ws_o + row * n_split * D;
  float m_lane = -INFINITY;
  for (int i = lane; i < n_split; i += 64) m_lane = fmaxf(m_lane, ml[i].x);
  const float M = rows_max(group_max<16>(m_lane));
  float l_lane = 0.f;
  for (int i = lane; i < n_split; i += 64)
    if (ml[i].x != -INFINITY) l_lane += ml[i].y * __builtin_amdgcn_exp2f(ml[i].x - M);
  const float inv = 1.f / rows_sum(group_sum<16>(l_lane));
  constexpr int E = D >= 64 ? D / 64 : 1;     // output dims per lane
  const bool has = D >= 64 || lane < D;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int c = 0; c < n_split; c += 64) {     // 64 ranges per round
    float w = 0.f;
    if (c + lane < n_split && ml[c + lane].x != -INFINITY) w = __builtin_amdgcn_exp2f(ml[c + lane].x - M);
    const int n = min(64, n_split - c);
    for (int j0 = 0; j0 < n; j0 += 8) {
      float x[8][E];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e)
          x[u][e] = (has && j0 + u < n) ? po[(size_t)(c + j0 + u) * D + lane * E + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j0 + u));
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(wu, wu > 0.f ? x[u][e] : 0.f, acc[e]);
      }
    }
  }
  if (has) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const size_t o = row * D + lane * E + e;
      const float v = acc[e] * inv;
      if constexpr (ElemBytes<PfComputeT<T>>::value == 4) {
        reinterpret_cast<float*>(a.out)[o] = v;
      } else {
        reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

template <typename T, int D, int G>
int launch_prefill(PrefillArgs a, int n_seqs, int max_chunk, hipStream_t st) {
  using S = PfShape<PfComputeT<T>, D, G>;
  a.n_qt = (max_chunk + S::MP - 1) / S::MP;
  a.n_work = a.n_qt * a.n_split * a.hkv * n_seqs;
  const int grid = (a.n_work + a.n_xcd - 1) / a.n_xcd * a.n_xcd;   // whole XCD rounds
  hipLaunchKernelGGL((prefill_attention_kernel<T, D, G>), dim3(grid), dim3(kPfThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return KVC_ERR_LAUNCH;
  if (a.n_split > 1) {
    hipLaunchKernelGGL((prefill_merge_kernel<T, D>), dim3((unsigned)a.total * a.hkv * G), dim3(64), 0,
                       st, a, a.hkv * G);
  }
  return launch_status();
}

template <typename T, int D>
int prefill_g(const PrefillArgs& a, int G, int n, int mc, hipStream_t st) {
  switch (G) {
    case 1: return launch_prefill<T, D, 1>(a, n, mc, st);
    case 2: return launch_prefill<T, D, 2>(a, n, mc, st);
    case 4: return launch_prefill<T, D, 4>(a, n, mc, st);
    case 8: return launch_prefill<T, D, 8>(a, n, mc, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

int dispatch_prefill(const PrefillArgs& a, int dtype, int D, int G, int n, int mc, hipStream_t st) {
  if (dtype == KVC_F32) {
    switch (D) {
      case 16: return prefill_g<float, 16>(a, G, n, mc, st);
      case 32: return prefill_g<float, 32>(a, G, n, mc, st);
      case 64: return prefill_g<float, 64>(a, G, n, mc, st);
      case 128: return prefill_g<float, 128>(a, G, n, mc, st);
    }
  } else if (dtype == KVC_BF16) {
    switch (D) {
      case 32: return prefill_g<bf16_tag, 32>(a, G, n, mc, st);
      case 64: return prefill_g<bf16_tag, 64>(a, G, n, mc, st);
      case 128: return prefill_g<bf16_tag, 128>(a, G, n, mc, st);
    }
  } else {
    switch (D) {
      case 64: return prefill_g<fp8_tag, 64>(a, G, n, mc, st);
      case 128: return prefill_g<fp8_tag, 128>(a, G, n, mc, st);
    }
  }
  return KVC_ERR_UNSUPPORTED;
}

// Key-range splits: when the query tiles alone give fewer than kPfTargetWork
// workgroups (a short chunk over a long cached prefix, such as the part of a
// prompt left after a prefix-cache hit), each query tile's keys are split into
// ranges of at least kPfMinSplitTiles tiles, and a merge combines the partials.
constexpr int kPfTargetWork = 512;
constexpr int kPfMinSplitTiles = 4;
constexpr int kPfMaxSplit = 32;

struct PfSplit {
  int n_split;
  int split_tiles;
};

PfSplit prefill_split(int n_seqs, int max_chunk, int max_ctx, int hkv, int G) {
  const int64_t n_qt = ceil_div(max_chunk, kRows / G);
  const int64_t base = n_qt * hkv * n_seqs;
  const int max_tiles = (int)ceil_div(max_ctx, kKeyTile);
  int n = 1;
  if (max_ctx > 0 && base < kPfTargetWork)
    n = (int)std::min<int64_t>(ceil_div(kPfTargetWork, base), max_tiles / kPfMinSplitTiles);
  n = std::max(1, std::min(n, kPfMaxSplit));
  if (n == 1) return {1, 1 << 30};
  const int tiles = (int)ceil_div(max_tiles, n);
  return {(int)ceil_div(max_tiles, tiles), tiles};
}

size_t prefill_ws_bytes(const PfSplit& sp, int total, int Hq, int D) {
  if (sp.n_split <= 1) return 0;
  return (size_t)total * Hq * sp.n_split * ((size_t)D * 4 + 8);
}

static int prefill_entry(const kvc_cache* cache, const void* q, const void* k, const void* v,
                         int32_t n_seqs, const int32_t* cu_chunk_lens, const int32_t* prefix_lens,
                         int32_t total_tokens, int32_t max_chunk_len, int32_t max_context_len,
                         const int32_t* block_table, int32_t max_blocks, int32_t Hq,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (n_seqs < 0 || total_tokens < 0 || max_chunk_len < 0 || max_blocks < 0 || Hq <= 0)
    return KVC_ERR_SHAPE;
  if (Hq % cache->num_kv_heads != 0) return KVC_ERR_SHAPE;
  const int G = Hq / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_tokens == 0 || max_chunk_len == 0) return KVC_OK;
  if (cache->num_blocks < 1) return KVC_ERR_SHAPE;   // a chunk needs somewhere to go
  if (!q || !k || !v || !cu_chunk_lens || !prefix_lens || !block_table || !out) return KVC_ERR_NULL;
  PfSplit sp{1, 1 << 30};
  if (max_context_len >= 0) {
    if (max_context_len < max_chunk_len) return KVC_ERR_SHAPE;
    sp = prefill_split(n_seqs, max_chunk_len, max_context_len, cache->num_kv_heads, G);
  }
  const size_t need = prefill_ws_bytes(sp, total_tokens, Hq, cache->head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KVC_ERR_WORKSPACE;
  if (!cache_aligned(cache) || !all_aligned(16, q, k, v, out, workspace) ||
      !all_aligned(4, cu_chunk_lens, prefix_lens, block_table))
    return KVC_ERR_ALIGN;
  const DeviceInfo dev = device_info();
  if (dev.cus == 0) return KVC_ERR_LAUNCH;
  hipStream_t s = as_stream(stream);
  st = launch_chunk_append(cache, k, v, n_seqs, cu_chunk_lens, prefix_lens, total_tokens,
                           max_chunk_len, block_table, max_blocks, s);
  if (st != KVC_OK) return st;
  PrefillArgs a;
  a.q = q;
  a.kc = cache->k_cache;
  a.vc = cache->v_cache;
  a.cu = cu_chunk_lens;
  a.prefix = prefix_lens;
  a.bt = block_table;
  a.out = out;
  a.err = cache->err_flag;
  a.hkv = cache->num_kv_heads;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = max_blocks;
  a.total = total_tokens;
  a.max_chunk = max_chunk_len;
  a.n_split = sp.n_split;
  a.split_tiles = sp.split_tiles;
  a.n_cus = dev.cus;
  a.n_xcd = dev.xcds;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.ks = cache->k_scale;
  a.vs = cache->v_scale;
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_ml = need > 0 ? reinterpret_cast<float2*>(reinterpret_cast<uint8_t*>(workspace) +
                                                  (size_t)total_tokens * Hq * sp.n_split *
                                                      cache->head_dim * 4)
                     : nullptr;
  return dispatch_prefill(a, cache->dtype, cache->head_dim, G, n_seqs, max_chunk_len, s);
}

}  // namespace kvc

extern "C" size_t kvc_prefill_workspace_bytes(int32_t n_seqs, int32_t total_tokens,
                                              int32_t max_chunk_len, int32_t max_context_len,
                                              int32_t Hq, int32_t num_kv_heads, int32_t head_dim) {
  if (n_seqs <= 0 || total_tokens <= 0 || max_chunk_len <= 0 || max_context_len < max_chunk_len ||
      Hq <= 0 || num_kv_heads <= 0 || head_dim <= 0 || Hq % num_kv_heads != 0)
    return 0;
  const kvc::PfSplit sp =
      kvc::prefill_split(n_seqs, max_chunk_len, max_context_len, num_kv_heads, Hq / num_kv_heads);
  return kvc::prefill_ws_bytes(sp, total_tokens, Hq, head_dim);
}

extern "C" int kvc_chunked_prefill_attention_split(
    const kvc_cache* cache, const void* q, const void* k, const void* v, int32_t n_seqs,
    const int32_t* cu_chunk_lens, const int32_t* prefix_lens, int32_t total_tokens,
    int32_t max_chunk_len, int32_t max_context_len, const int32_t* block_table, int32_t max_blocks,
    int32_t Hq, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (max_context_len < 0) return KVC_ERR_SHAPE;
  return kvc::prefill_entry(cache, q, k, v, n_seqs, cu_chunk_lens, prefix_lens, total_tokens,
                            max_chunk_len, max_context_len, block_table, max_blocks, Hq,
                            softmax_scale, out, workspace, workspace_bytes, stream);
}

extern "C" int kvc_chunked_prefill_attention(const kvc_cache* cache, const void* q, const void* k,
                                             const void* v, int32_t n_seqs, const int32_t* cu_chunk_lens,
                                             const int32_t* prefix_lens, int32_t total_tokens,
                                             int32_t max_chunk_len, const int32_t* block_table,
                                             int32_t max_blocks, int32_t Hq, float softmax_scale,
                                             void* out, void* stream) {
  return kvc::prefill_entry(cache, q, k, v, n_seqs, cu_chunk_lens, prefix_lens, total_tokens,
                            max_chunk_len, -1, block_table, max_blocks, Hq, softmax_scale, out,
                            nullptr, 0, stream);
}
