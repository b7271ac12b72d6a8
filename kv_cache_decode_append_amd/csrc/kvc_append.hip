// Slot mapping and KV append.
//
// A decode step appends the new position's key and value to the cache before
// attending over everything stored (aiwithghost.com "KV cache and continuous
// batching: 1,000 people ask AI", section "What does a KV cache keep?";
// daviddominguez.dev "The KV cache and prefix caching", section "What prefill
// stores and decode reads"). The cache is paged: fixed 16-token blocks reached
// through a per-sequence block table (daviddominguez.dev, same section and
// section "A prefix already in the cache can skip its prefill").
//
// Both kernels are pure integer work / byte copies: bit-exact by construction.
// The append is HBM-bound and tiny (one 16-byte chunk per lane, each token row
// of one head is `head_dim * elem` contiguous bytes on both sides).

#include "kvc_append.h"
#include "kvc_device.h"
#include "kvc_host.h"

namespace kvc {

__global__ void slot_mapping_kernel(const int32_t* __restrict__ block_table, int32_t n_seqs,
                                    int32_t max_blocks,
                                    int32_t num_blocks, const int32_t* __restrict__ seq_ids,
                                    const int32_t* __restrict__ positions, int32_t T,
                                    int64_t* __restrict__ slots, int32_t* err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int32_t p = positions[t];
  int64_t slot = -1;
  const int32_t sid = seq_ids[t];
  if (p >= 0) {
    const int32_t lb = p >> 4;
    if (lb >= max_blocks || sid < 0 || sid >= n_seqs) {
      flag_error(err, KVC_DEVERR_CONTEXT);
    } else {
      const int32_t blk = block_table[(int64_t)sid * max_blocks + lb];
      if (blk < 0 || blk >= num_blocks)
        flag_error(err, KVC_DEVERR_BLOCK_ID);
      else
        slot = (int64_t)blk * 16 + (p & 15);
    }
  }
  slots[t] = slot;
}

// One 16-byte chunk of K and of V per thread.
// chunk id -> (token t, kv head h, chunk c), rows are `nc` chunks long.
__global__ void kv_append_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                 const int64_t* __restrict__ slots,
                                 const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                 int64_t n_chunks, int32_t hkv, int32_t nc,
                                 int64_t num_slots, int32_t* err) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_chunks) return;
  const int64_t row = i / nc;          // (t, h)
  const int32_t c = (int32_t)(i - row * nc);
  const int64_t t = row / hkv;
  const int32_t h = (int32_t)(row - t * hkv);
  const int64_t slot = slots[t];
  if (slot < 0) return;
  if (slot >= num_slots) {
    if (h == 0 && c == 0) flag_error(err, KVC_DEVERR_SLOT);
    return;
  }
  const int64_t blk = slot >> 4, off = slot & 15;
  const int64_t row_bytes = (int64_t)nc * 16;
  const int64_t dst = ((blk * hkv + h) * 16 + off) * row_bytes + (int64_t)c * 16;
  const int64_t src = i * 16;
  *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(k + src);
  *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(v + src);
}

// fp8 cache: one 8-value chunk of a (token, kv head) row per thread. The NCB =
// head_dim / 8 threads of a row (an aligned group of 8 or 16 lanes) find the
// row's largest magnitude together, then each codes its 8 values with the
// row's scale (amax / 448; a row below kZeroRowAmax is stored as zeros) and
// the first stores the scale.
template <int NCB>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, const int64_t* __restrict__ slots, const uint8_t* __restrict__ k,
    const uint8_t* __restrict__ v, int64_t n_chunks, int32_t hkv, int64_t num_slots,
    int32_t* err) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool in = i < n_chunks;
  const int64_t row = i / NCB;            // (t, h)
  const int32_t c = (int32_t)(i % NCB);
  const int64_t t = row / hkv;
  const int32_t h = (int32_t)(row - t * hkv);
  const int64_t slot = in ? slots[t] : -1;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const u32x4 kx = in ? *reinterpret_cast<const u32x4*>(k + i * 16) : zero;
  const u32x4 vx = in ? *reinterpret_cast<const u32x4*>(v + i * 16) : zero;
  // every lane of the group takes part in the reductions, so no early exit above
  const float ka = group_max<NCB>(bf16x8_amax(kx));
  const float va = group_max<NCB>(bf16x8_amax(vx));
  if (!in || slot < 0) return;
  if (slot >= num_slots) {
    if (h == 0 && c == 0) flag_error(err, KVC_DEVERR_SLOT);
    return;
  }
  const int64_t prow = ((slot >> 4) * hkv + h) * 16 + (slot & 15);   // row of the pools
  const bool kz = !(ka >= kZeroRowAmax), vz = !(va >= kZeroRowAmax);
  const u32x2 kq = kz ? u32x2{0u, 0u} : bf16x8_to_e4m3x8(kx, kE4M3Max / ka);
  const u32x2 vq = vz ? u32x2{0u, 0u} : bf16x8_to_e4m3x8(vx, kE4M3Max / va);
  *reinterpret_cast<u32x2*>(kc + prow * (NCB * 8) + c * 8) = kq;
  *reinterpret_cast<u32x2*>(vc + prow * (NCB * 8) + c * 8) = vq;
  if (c == 0) {
    ks[prow] = kz ? 0.f : ka / kE4M3Max;
    vs[prow] = vz ? 0.f : va / kE4M3Max;
  }
}

// Prefill-chunk write: token r of sequence s (r < C_s) goes to position
// prefix_s + r. grid = (ceil(max_chunk * hkv * nc / 256), n_seqs).
__global__ void chunk_append_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
                                    const int32_t* __restrict__ block_table, int32_t max_blocks,
                                    int32_t num_blocks, int32_t hkv, int32_t nc, int32_t total,
                                    int32_t max_chunk, int32_t* err) {
  const int s = blockIdx.y;
  const int32_t t0 = cu[s], C = cu[s + 1] - t0, p0 = prefix[s];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (!chunk_ok(t0, C, p0, total, max_chunk)) {
    if (i == 0) flag_error(err, KVC_DEVERR_CONTEXT);
    return;
  }
  if (i >= (int64_t)C * hkv * nc) return;
  const int64_t row = i / nc;
  const int32_t c = (int32_t)(i - row * nc);
  const int32_t r = (int32_t)(row / hkv);
  const int32_t h = (int32_t)(row - (int64_t)r * hkv);
  const int bad = chunk_append_one(kc, vc, k, v, block_table + (int64_t)s * max_blocks, max_blocks,
                                   num_blocks, hkv, nc, t0, p0, r, h, c);
  if (bad && h == 0 && c == 0) flag_error(err, bad);
}

// fp8 cache: the chunk rows quantised as kv_append_fp8_kernel does, one 8-value
// chunk per thread, the NCB threads of a row reducing its amax together.
// grid = (ceil(max_chunk * hkv * NCB / 256), n_seqs).
template <int NCB>
__global__ __launch_bounds__(256) void chunk_append_fp8_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ block_table, int32_t max_blocks, int32_t num_blocks, int32_t hkv,
    int32_t total, int32_t max_chunk, int32_t* err) {
  const int s = blockIdx.y;
  const int32_t t0 = cu[s], C = cu[s + 1] - t0, p0 = prefix[s];
  const bool ok = chunk_ok(t0, C, p0, total, max_chunk);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / NCB;                 // (r, h)
  const int32_t c = (int32_t)(i % NCB);
  const int32_t r = (int32_t)(row / hkv);
  const int32_t h = (int32_t)(row - (int64_t)r * hkv);
  // every lane of a row's group takes part in its reduction: no early exit
  const int bad = chunk_append_fp8_one<NCB>(kc, vc, ks, vs, k, v,
                                            block_table + (int64_t)s * max_blocks, max_blocks,
                                            num_blocks, hkv, t0, p0, r, h, c, ok && r < C);
  if (!ok) {
    if (i == 0) flag_error(err, KVC_DEVERR_CONTEXT);
    return;
  }
  if (bad && h == 0 && c == 0) flag_error(err, bad);
}

int launch_chunk_append(const kvc_cache* c, const void* k, const void* v, int32_t n_seqs,
                        const int32_t* cu, const int32_t* prefix, int32_t total, int32_t max_chunk,
                        const int32_t* block_table, int32_t max_blocks, hipStream_t st) {
  if (c->dtype == KVC_FP8) {
    const int ncb = c->head_dim / 8;
    const int64_t per_seq = (int64_t)max_chunk * c->num_kv_heads * ncb;
    if (per_seq == 0 || n_seqs == 0) return KVC_OK;
    auto kern = ncb == 16 ? chunk_append_fp8_kernel<16> : chunk_append_fp8_kernel<8>;
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(per_seq, 256), (unsigned)n_seqs), dim3(256), 0,
                       st, (uint8_t*)c->k_cache, (uint8_t*)c->v_cache, c->k_scale, c->v_scale,
                       (const uint8_t*)k, (const uint8_t*)v, cu, prefix, block_table, max_blocks,
                       c->num_blocks, c->num_kv_heads, total, max_chunk, c->err_flag);
    return launch_status();
  }
  const int nc = c->head_dim * dtype_bytes(c->dtype) / 16;
  const int64_t per_seq = (int64_t)max_chunk * c->num_kv_heads * nc;
  if (per_seq == 0 || n_seqs == 0) return KVC_OK;
  dim3 grid((unsigned)ceil_div(per_seq, 256), (unsigned)n_seqs);
  hipLaunchKernelGGL(chunk_append_kernel, grid, dim3(256), 0, st, (uint8_t*)c->k_cache,
                     (uint8_t*)c->v_cache, (const uint8_t*)k, (const uint8_t*)v, cu, prefix,
                     block_table, max_blocks, c->num_blocks, c->num_kv_heads, nc, total, max_chunk,
                     c->err_flag);
  return launch_status();
}

}  // namespace kvc

extern "C" int kvc_slot_mapping(const int32_t* block_table, int32_t n_seqs, int32_t max_blocks,
                                int32_t num_blocks, const int32_t* seq_ids, const int32_t* positions, int32_t T,
                                int32_t block_size, int64_t* slot_mapping, int32_t* err_flag,
                                void* stream) {
  if (T < 0 || n_seqs < 0 || max_blocks < 0 || num_blocks < 0) return KVC_ERR_SHAPE;
  if (block_size != 16) return KVC_ERR_UNSUPPORTED;
  if (T == 0) return KVC_OK;
  if (!block_table || !seq_ids || !positions || !slot_mapping) return KVC_ERR_NULL;
  if (!kvc::all_aligned(4, block_table, seq_ids, positions, err_flag) ||
      !kvc::aligned_to(slot_mapping, 8))
    return KVC_ERR_ALIGN;
  hipLaunchKernelGGL(kvc::slot_mapping_kernel, dim3((unsigned)kvc::ceil_div(T, 256)), dim3(256), 0,
                     kvc::as_stream(stream), block_table, n_seqs, max_blocks, num_blocks, seq_ids,
                     positions, T, slot_mapping, err_flag);
  return kvc::launch_status();
}

extern "C" int kvc_kv_append(const kvc_cache* cache, const int64_t* slot_mapping, const void* k,
                             const void* v, int32_t T, void* stream) {
  int st = kvc::check_cache(cache);
  if (st != KVC_OK) return st;
  if (T < 0) return KVC_ERR_SHAPE;
  if (T == 0) return KVC_OK;
  if (!slot_mapping || !k || !v) return KVC_ERR_NULL;
  if (!kvc::cache_aligned(cache) || !kvc::aligned_to(slot_mapping, 8) || !kvc::all_aligned(16, k, v))
    return KVC_ERR_ALIGN;
  if (cache->dtype == KVC_FP8) {
    const int ncb = cache->head_dim / 8;
    const int64_t n = (int64_t)T * cache->num_kv_heads * ncb;
    auto kern = ncb == 16 ? kvc::kv_append_fp8_kernel<16> : kvc::kv_append_fp8_kernel<8>;
    hipLaunchKernelGGL(kern, dim3((unsigned)kvc::ceil_div(n, 256)), dim3(256), 0,
                       kvc::as_stream(stream), (uint8_t*)cache->k_cache, (uint8_t*)cache->v_cache,
                       cache->k_scale, cache->v_scale, slot_mapping, (const uint8_t*)k,
                       (const uint8_t*)v, n, cache->num_kv_heads,
                       (int64_t)cache->num_blocks * 16, cache->err_flag);
    return kvc::launch_status();
  }
  const int nc = cache->head_dim * kvc::dtype_bytes(cache->dtype) / 16;
  const int64_t n_chunks = (int64_t)T * cache->num_kv_heads * nc;
  hipLaunchKernelGGL(kvc::kv_append_kernel, dim3((unsigned)kvc::ceil_div(n_chunks, 256)), dim3(256),
                     0, kvc::as_stream(stream), (uint8_t*)cache->k_cache, (uint8_t*)cache->v_cache,
                     slot_mapping, (const uint8_t*)k, (const uint8_t*)v, n_chunks,
                     cache->num_kv_heads, nc, (int64_t)cache->num_blocks * 16, cache->err_flag);
  return kvc::launch_status();
}
