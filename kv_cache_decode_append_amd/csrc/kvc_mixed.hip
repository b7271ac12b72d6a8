// One launch for a continuous-batching step that mixes decode rows and prefill
// chunks.
//
// Continuous batching rebuilds the batch every step, so a step holds rows that
// decode one token next to requests that start with their prefill
// (aiwithghost.com "KV cache and continuous batching: 1,000 people ask AI",
// section "How does continuous batching share the server?"), and with decode
// first the prefill chunks fill a token budget beside the decode rows
// (gouthm.com "The KV cache is not your bottleneck", section "The fix that
// mattered"). Two launches (decode, then prefill) serialise the HBM-bound
// decode and the MFMA-bound prefill and leave the chip idle behind each one's
// slowest workgroup. Here one persistent kernel takes work items from a queue
// in device memory:
//
//   phase 0   the prefill chunks' K/V go into the cache, 64 rows per item;
//             for a large decode batch, one more item first orders the decode
//             rows longest first (by the power of two of their block count);
//   then      prefill items, one per (query tile, kv head, chunk), later
//             query tiles (more keys) first, and decode items, one per (kv
//             head, row), each writing the row's new K/V and then walking its
//             whole context, so no partial results need merging across
//             workgroups. Prefill items come first (the largest items start
//             earliest), and the decode items fill in behind them; HBM-bound
//             decode items and MFMA-bound prefill items then run side by side
//             on different compute units.
//
// Workgroups are 8 waves (the prefill item's shape; a decode item spreads a
// row's blocks over the 8 waves) and the grid is at most one resident wave of
// workgroups. Workgroup i starts with item i and then takes items from the
// queue (with a workgroup per item there is no queue, and without phase-0
// items no atomic at all). A prefill item, and a decode item when the rows are ordered, first
// waits until every phase-0 item is done (they write what it reads); phase-0
// items have the lowest indices, so they belong to workgroups dispatched
// before any that wait, and the wait is bounded anyway. The queue header is
// reset by the last workgroup to leave.

#include <algorithm>
#include <atomic>

#include "kvc_decode_item.h"
#include "kvc_host.h"
#include "kvc_prefill_item.h"

namespace kvc {

constexpr int kMixWaves = 8;
constexpr int kMixThreads = kMixWaves * 64;
constexpr int kMixMaxDecode = 4096;      // decode rows per call (their order is kept in LDS)
constexpr int kAppendRows = 64;          // prefill chunk rows per phase-0 item
constexpr int kSpinLimit = 1 << 20;      // phase-0 wait: ~0.2 s of s_sleep before giving up
static_assert(kMixThreads == kPfThreads, "the prefill item needs the whole workgroup");

struct MixedHeader {
  int32_t next;         // next item to hand out
  int32_t phase0_done;  // phase-0 items finished
  int32_t exited;       // workgroups that left the loop
};

struct MixedArgs {
  DecodeArgs dec;       // n_seqs = decode rows, one partition per row
  PrefillArgs pf;       // n_split = 1
  const uint8_t* k_pf;  // the chunks' K/V (packed rows)
  const uint8_t* v_pf;
  const uint8_t* k_new; // the decode rows' new K/V, [n_dec][hkv][D]
  const uint8_t* v_new;
  int32_t plan;         // 1: phase-0 item 0 orders the decode rows
  int32_t nc;           // 16-byte chunks per new K/V row (bf16 rows for an fp8 cache)
  MixedHeader* hdr;
  int32_t* dec_order;   // [n_dec]: decode rows, longest first (when planned)
  int32_t n_dec;
  int32_t n_pf;
  int32_t n_slices;     // phase-0 items per chunk
  int32_t n_phase0;     // plan + n_pf * n_slices
  int32_t n_pf_items;   // n_qt * hkv * n_pf
  int32_t n_dec_items;  // hkv * n_dec
  int32_t one_each;     // the grid has a workgroup per item: no queue
};

// Item 0 of phase 0: the decode rows in decreasing order of
// floor(log2(blocks)) (a coarse longest-first order; rows with the same key
// may come in any order, which changes no result).
__device__ __forceinline__ void plan_decode(const MixedArgs& m, int32_t* scratch) {
  const int tid = threadIdx.x;
  int32_t* cnt = scratch;          // [32] rows per key
  int32_t* fill = scratch + 32;    // [32] rows placed per key
  if (tid < 64) scratch[tid] = 0;
  __syncthreads();
  constexpr int PER = kMixMaxDecode / kMixThreads;   // rows per thread
  int key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = tid * PER + j;
    key[j] = -1;
    if (b < m.n_dec) {
      const int nblk = (effective_ctx(m.dec, b, false) + 15) >> 4;
      key[j] = 31 - __builtin_clz((unsigned)max(nblk, 1));
      atomicAdd(&cnt[key[j]], 1);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (key[j] < 0) continue;
    int start = 0;
    for (int k = 31; k > key[j]; --k) start += cnt[k];
    m.dec_order[start + atomicAdd(&fill[key[j]], 1)] = tid * PER + j;
  }
}

// The new K/V of decode row b for kv head kvh at position context_len - 1,
// written by the decode item itself before it reads the row (a workgroup
// barrier orders the two); an fp8 cache gets the row's codes and scale, made
// by the first D / 8 lanes together. A row with an empty context holds no token,
// and a row whose length exceeds the bounds gets no append (the decode item
// flags it).
template <typename T, int D>
__device__ __forceinline__ void append_decode_row(const MixedArgs& m, int b, int kvh, int tid) {
  const DecodeArgs& a = m.dec;
  if (tid < m.nc) {
    bool ok;
    const int ctx = effective_ctx(a, b, false, &ok);
    if (ok && ctx >= 1) {
      const int32_t* bt_row = a.bt + (size_t)b * a.max_blocks;
      int bad;
      if constexpr (std::is_same_v<T, fp8_tag>)
        bad = chunk_append_fp8_one<D / 8>((uint8_t*)a.kc, (uint8_t*)a.vc, a.ks, a.vs, m.k_new,
                                          m.v_new, bt_row, a.max_blocks, a.num_blocks, a.hkv, b,
                                          ctx - 1, 0, kvh, tid, true);
      else
        bad = chunk_append_one((uint8_t*)a.kc, (uint8_t*)a.vc, m.k_new, m.v_new, bt_row,
                               a.max_blocks, a.num_blocks, a.hkv, m.nc, b, ctx - 1, 0, kvh, tid);
      if (bad && tid == 0) flag_error(a.err, bad);
    }
  }
  __threadfence_block();
  __syncthreads();
}

// Phase 0: rows [64 * slice, 64 * slice + 64) of prefill chunk s (coded with
// their row scales for an fp8 cache: a row's D / 8 chunks are consecutive
// indices, so they sit in one aligned lane group of every pass).
template <typename T, int D>
__device__ __forceinline__ void append_slice(const MixedArgs& m, int idx) {
  const PrefillArgs& p = m.pf;
  const int s = idx / m.n_slices, slice = idx % m.n_slices;
  const int t0 = p.cu[s], C = p.cu[s + 1] - t0, p0 = p.prefix[s];
  if (!chunk_ok(t0, C, p0, p.total, p.max_chunk)) return;   // the prefill item flags it
  const int r0 = slice * kAppendRows, r1 = min(C, r0 + kAppendRows);
  const int per_row = p.hkv * m.nc;
  const int32_t* bt_row = p.bt + (size_t)s * p.max_blocks;
  int bad = 0;
  for (int i = threadIdx.x; i < (r1 - r0) * per_row; i += kMixThreads) {
    const int r = r0 + i / per_row, hc = i % per_row;
    if constexpr (std::is_same_v<T, fp8_tag>)
      bad |= chunk_append_fp8_one<D / 8>((uint8_t*)p.kc, (uint8_t*)p.vc, const_cast<float*>(p.ks),
                                         const_cast<float*>(p.vs), m.k_pf, m.v_pf, bt_row,
                                         p.max_blocks, p.num_blocks, p.hkv, t0, p0, r, hc / m.nc,
                                         hc % m.nc, true);
    else
      bad |= chunk_append_one((uint8_t*)p.kc, (uint8_t*)p.vc, m.k_pf, m.v_pf, bt_row, p.max_blocks,
                              p.num_blocks, p.hkv, m.nc, t0, p0, r, hc / m.nc, hc % m.nc);
  }
  if (bad) flag_error(p.err, bad);
}

// The arguments, read from the kernel-argument segment through a pointer the
// compiler cannot see through: each use loads what it needs where it runs, so
// the persistent loop does not keep both item kinds' arguments live in scalar
// registers across iterations (that pushed the kernel past its registers).
__device__ __forceinline__ const MixedArgs* fresh_args() {
  using KArgs = const __attribute__((address_space(4))) MixedArgs;
  KArgs* kp = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return (const MixedArgs*)kp;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kMixThreads) void mixed_step_kernel(MixedArgs) {
  using DS = DecodeShape<ComputeT<T>, D, G, kMixWaves>;
  using PS = PfShape<PfComputeT<T>, D, G>;
  constexpr int WORK = DS::SMEM > PS::SMEM ? DS::SMEM : PS::SMEM;
  __shared__ __attribute__((aligned(16))) uint8_t smem[WORK + kMixMaxDecode * 4 + 64];
  int32_t* order_lds = reinterpret_cast<int32_t*>(smem + WORK);
  int32_t* ctl = order_lds + kMixMaxDecode;       // [0] the fetched item
  const int tid = threadIdx.x;
  bool open = false;          // phase 0 seen complete (uniform over the workgroup)
  bool first = true;
  for (;;) {
    const MixedArgs& m = *fresh_args();
    int item = blockIdx.x;
    if (!first) {
      if (m.one_each) break;
      if (tid == 0) ctl[0] = (int)gridDim.x + atomicAdd(&m.hdr->next, 1);
      __syncthreads();
      item = ctl[0];
    }
    first = false;
    if (item < m.n_phase0) {
      if (m.plan && item == 0)
        plan_decode(m, reinterpret_cast<int32_t*>(smem));
      else
        append_slice<T, D>(m, item - m.plan);
      __threadfence();                             // publish this item's writes
      __syncthreads();
      if (tid == 0) atomicAdd(&m.hdr->phase0_done, 1);
    } else {
      // item -> (prefill or decode, index in that list)
      const int k = item - m.n_phase0;
      const int64_t n_pf = m.n_pf_items, n_all = n_pf + m.n_dec_items;
      if (k >= n_all) break;
      // prefill items first: the largest items (late query tiles over long
      // prefixes) start earliest and the short decode items fill the tail
      const bool is_pf = k < n_pf;
      const int idx = is_pf ? k : k - (int)n_pf;
      if (!open && (is_pf || m.plan)) {
        if (tid == 0) {
          int spins = 0;
          while (__hip_atomic_load(&m.hdr->phase0_done, __ATOMIC_ACQUIRE,
                                   __HIP_MEMORY_SCOPE_AGENT) < m.n_phase0) {
            __builtin_amdgcn_s_sleep(4);
            if (++spins == kSpinLimit) {
              flag_error(m.dec.err, KVC_DEVERR_QUEUE);
              break;
            }
          }
        }
        __syncthreads();
        __threadfence();                           // see every phase-0 write
        if (m.plan)
          for (int i = tid; i < m.n_dec; i += kMixThreads) order_lds[i] = m.dec_order[i];
        __syncthreads();
        open = true;
      }
      const int hkv = m.dec.hkv;
      // the thread index, opaque here too, so that nothing derived from it is
      // hoisted out of the loop and held in vector registers across items
      int my_tid = tid;
      asm volatile("" : "+v"(my_tid));
      if (is_pf) {
        // costliest chunks first (at most 64 chunks, else in index order), and
        // in a chunk later query tiles first: index -> (chunk, qt descending,
        // kv head)
        const MixedArgs& mi = *fresh_args();
        const int per = hkv * mi.pf.n_qt;
        const int rank = idx / per, qt = mi.pf.n_qt - 1 - (idx % per) / hkv, kvh = idx % hkv;
        const int s = mi.n_pf <= kMaxRankedSeqs ? seq_with_cost_rank(mi.pf, mi.n_pf, rank) : rank;
        prefill_item<T, D, G>(mi.pf, qt + mi.pf.n_qt * (kvh + hkv * s), smem, my_tid);
      } else {
        const MixedArgs& mi = *fresh_args();
        const int b = mi.plan ? order_lds[idx / hkv] : idx / hkv, kvh = idx % hkv;
        append_decode_row<T, D>(mi, b, kvh, my_tid);
        decode_item<T, D, G, kMixWaves, true, false>(mi.dec, kvh, b, 0, smem, my_tid);
      }
    }
    __syncthreads();                               // LDS and ctl free for the next item
  }
  const MixedArgs& m = *fresh_args();
  if (tid == 0 && (!m.one_each || m.n_phase0 > 0)) {
    if (atomicAdd(&m.hdr->exited, 1) == (int)gridDim.x - 1) {
      atomicExch(&m.hdr->next, 0);
      atomicExch(&m.hdr->phase0_done, 0);
      atomicExch(&m.hdr->exited, 0);
    }
  }
}

// ---- host ----

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: the 256-byte queue header, then the decode row order.
size_t mixed_ws_bytes(int n_dec) { return 256 + align256((size_t)n_dec * 4); }

template <typename T, int D, int G>
int launch_mixed(const MixedArgs& m, int64_t n_items_max, hipStream_t st) {
  // one resident wave of workgroups: CUs x workgroups per CU, cached per device
  // (as their product; calls from several host threads may race to fill an
  // entry, with the same value)
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return KVC_ERR_LAUNCH;
  int resident = cached[dev].load(std::memory_order_relaxed);
  if (resident == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mixed_step_kernel<T, D, G>,
                                                     kMixThreads, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
      return KVC_ERR_LAUNCH;
    resident = cus * per_cu;
    cached[dev].store(resident, std::memory_order_relaxed);
  }
  const int64_t grid = std::min<int64_t>(n_items_max, (int64_t)resident);
  MixedArgs mm = m;
  mm.one_each = grid == n_items_max ? 1 : 0;
  hipLaunchKernelGGL((mixed_step_kernel<T, D, G>), dim3((unsigned)grid), dim3(kMixThreads), 0, st,
                     mm);
  return launch_status();
}

// Instantiated where both item bodies fit the 256 registers a lane has at 8
// waves per workgroup without spilling: bf16 and fp8 head_dim 64 and 128,
// fp32 head_dim 32, with G <= 4.
template <typename T, int D>
int mixed_g(const MixedArgs& m, int G, int64_t n, hipStream_t st) {
  switch (G) {
    case 1: return launch_mixed<T, D, 1>(m, n, st);
    case 2: return launch_mixed<T, D, 2>(m, n, st);
    case 4: return launch_mixed<T, D, 4>(m, n, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

int dispatch_mixed(const MixedArgs& m, int dtype, int D, int G, int64_t n, hipStream_t st) {
  if (dtype == KVC_BF16) {
    if (D == 64) return mixed_g<bf16_tag, 64>(m, G, n, st);
    if (D == 128) return mixed_g<bf16_tag, 128>(m, G, n, st);
  } else if (dtype == KVC_FP8) {
    if (D == 64) return mixed_g<fp8_tag, 64>(m, G, n, st);
    if (D == 128) return mixed_g<fp8_tag, 128>(m, G, n, st);
  } else if (D == 32) {
    return mixed_g<float, 32>(m, G, n, st);
  }
  return KVC_ERR_UNSUPPORTED;
}

bool mixed_supported(int dtype, int D, int G) {
  const bool dim_ok = dtype == KVC_F32 ? D == 32 : (D == 64 || D == 128);
  return dim_ok && (G == 1 || G == 2 || G == 4);
}

}  // namespace kvc

extern "C" size_t kvc_mixed_workspace_bytes(int32_t n_decode, int32_t decode_max_context,
                                            int32_t Hq, int32_t num_kv_heads, int32_t head_dim) {
  if (n_decode < 0 || n_decode > kvc::kMixMaxDecode || decode_max_context < 0 || Hq <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || Hq % num_kv_heads != 0)
    return 0;
  return kvc::mixed_ws_bytes(n_decode);
}

extern "C" int kvc_mixed_step_attention(const kvc_cache* cache, const kvc_mixed_batch* bt,
                                        int32_t Hq, float softmax_scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  using namespace kvc;
  int st = check_cache(cache);
  if (st != KVC_OK) return st;
  if (!bt) return KVC_ERR_NULL;
  if (Hq <= 0 || Hq % cache->num_kv_heads != 0) return KVC_ERR_SHAPE;
  const int hkv = cache->num_kv_heads, D = cache->head_dim, G = Hq / hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KVC_ERR_UNSUPPORTED;
  const kvc_mixed_batch& b = *bt;
  if (b.n_decode < 0 || b.n_prefill < 0 || b.decode_max_blocks < 0 || b.decode_max_context < 0 ||
      b.prefill_total_tokens < 0 || b.prefill_max_chunk < 0 || b.prefill_max_blocks < 0)
    return KVC_ERR_SHAPE;
  if (b.n_decode > kMixMaxDecode) return KVC_ERR_UNSUPPORTED;
  if ((int64_t)b.decode_max_context > (int64_t)b.decode_max_blocks * 16) return KVC_ERR_SHAPE;
  const bool has_dec = b.n_decode > 0;
  const bool has_pf = b.n_prefill > 0 && b.prefill_total_tokens > 0 && b.prefill_max_chunk > 0;
  if (!mixed_supported(cache->dtype, D, G)) return KVC_ERR_UNSUPPORTED;
  if (!has_dec && !has_pf) return KVC_OK;
  if (has_dec && (!b.q_decode || !b.k_new || !b.v_new || !b.decode_block_table ||
                  !b.decode_context_lens || !b.out_decode))
    return KVC_ERR_NULL;
  if (has_pf) {
    if (!b.q_prefill || !b.k_prefill || !b.v_prefill || !b.cu_chunk_lens || !b.prefix_lens ||
        !b.prefill_block_table || !b.out_prefill)
      return KVC_ERR_NULL;
    if (cache->num_blocks < 1) return KVC_ERR_SHAPE;
  }
  const int n_dec = has_dec ? b.n_decode : 0;
  if (!workspace || workspace_bytes < mixed_ws_bytes(n_dec)) return KVC_ERR_WORKSPACE;
  if (!cache_aligned(cache) || !aligned_to(workspace, 16)) return KVC_ERR_ALIGN;
  if (has_dec && (!all_aligned(16, b.q_decode, b.k_new, b.v_new, b.out_decode) ||
                  !all_aligned(4, b.decode_block_table, b.decode_context_lens)))
    return KVC_ERR_ALIGN;
  if (has_pf && (!all_aligned(16, b.q_prefill, b.k_prefill, b.v_prefill, b.out_prefill) ||
                 !all_aligned(4, b.cu_chunk_lens, b.prefix_lens, b.prefill_block_table)))
    return KVC_ERR_ALIGN;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);

  MixedArgs m{};
  DecodeArgs& a = m.dec;
  a.q = b.q_decode;
  a.k_new = nullptr;         // written in phase 0
  a.v_new = nullptr;
  a.kc = cache->k_cache;
  a.vc = cache->v_cache;
  a.bt = b.decode_block_table;
  a.ctx_lens = b.decode_context_lens;
  a.out = b.out_decode;
  a.ws_o = nullptr;          // one partition per row: no partials
  a.ws_ml = nullptr;
  a.err = cache->err_flag;
  a.hkv = hkv;
  a.n_seqs = n_dec;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = b.decode_max_blocks;
  a.max_ctx = b.decode_max_context;
  a.part_blocks = 1 << 30;
  a.ks = cache->k_scale;      // fp8 row scales (null otherwise)
  a.vs = cache->v_scale;
  a.n_part = 1;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;

  PrefillArgs& p = m.pf;
  p.q = b.q_prefill;
  p.kc = cache->k_cache;
  p.vc = cache->v_cache;
  p.cu = b.cu_chunk_lens;
  p.prefix = b.prefix_lens;
  p.bt = b.prefill_block_table;
  p.out = b.out_prefill;
  p.err = cache->err_flag;
  p.hkv = hkv;
  p.num_blocks = cache->num_blocks;
  p.max_blocks = b.prefill_max_blocks;
  p.total = b.prefill_total_tokens;
  p.max_chunk = b.prefill_max_chunk;
  const int mp = kRows / G;
  p.n_qt = has_pf ? (int)ceil_div(b.prefill_max_chunk, mp) : 0;
  p.n_split = 1;
  p.split_tiles = 1 << 30;
  p.n_work = p.n_qt * hkv * (has_pf ? b.n_prefill : 0);
  p.scale_log2 = a.scale_log2;
  p.ws_o = nullptr;
  p.ws_ml = nullptr;
  p.ks = cache->k_scale;
  p.vs = cache->v_scale;

  m.k_pf = reinterpret_cast<const uint8_t*>(b.k_prefill);
  m.v_pf = reinterpret_cast<const uint8_t*>(b.v_prefill);
  m.k_new = reinterpret_cast<const uint8_t*>(b.k_new);
  m.v_new = reinterpret_cast<const uint8_t*>(b.v_new);
  // order the decode rows only when there are many more decode items than
  // workgroups and some row is long enough for its order to matter
  m.plan = (int64_t)n_dec * hkv > 2 * 256 && b.decode_max_context > 4096 ? 1 : 0;
  // 16-byte chunks of a new K/V row as passed in (bf16 rows for an fp8 cache)
  m.nc = D * (cache->dtype == KVC_FP8 ? 2 : dtype_bytes(cache->dtype)) / 16;
  m.hdr = reinterpret_cast<MixedHeader*>(ws);
  m.dec_order = reinterpret_cast<int32_t*>(ws + 256);
  m.n_dec = n_dec;
  m.n_pf = has_pf ? b.n_prefill : 0;
  m.n_slices = has_pf ? (int)ceil_div(b.prefill_max_chunk, kAppendRows) : 0;
  const int64_t n_phase0 = m.plan + (int64_t)m.n_pf * m.n_slices;
  const int64_t n_items_max = n_phase0 + p.n_work + (int64_t)n_dec * hkv;
  if (n_items_max > INT32_MAX / 2) return KVC_ERR_SHAPE;
  m.n_phase0 = (int)n_phase0;
  m.n_pf_items = p.n_work;
  m.n_dec_items = n_dec * hkv;
  return dispatch_mixed(m, cache->dtype, D, G, n_items_max, as_stream(stream));
}
