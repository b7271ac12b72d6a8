/*
 * kvc.h - paged KV-cache append, paged GQA decode attention and chunked-prefill
 * attention for AMD MI355X (gfx950). C ABI: plain pointers and sizes only.
 *
 * What the library computes (restated from the pages it follows):
 *   - A decode step computes one new position's query, key and value, appends
 *     the key and value to the cache and attends the new query over everything
 *     stored (aiwithghost.com "KV cache and continuous batching: 1,000 people ask
 *     AI", section "What does a KV cache keep?"; daviddominguez.dev "The KV cache
 *     and prefix caching", section "What prefill stores and decode reads").
 *   - The cache is held in fixed-size blocks reached through a per-sequence block
 *     table, not in one contiguous slab per request (daviddominguez.dev, same
 *     section, on the PagedAttention design); blocks hold 16 tokens
 *     (daviddominguez.dev, section "A prefix already in the cache can skip its
 *     prefill").
 *   - Several query heads share one key/value head (grouped-query attention,
 *     daviddominguez.dev, section "What prefill stores and decode reads").
 *   - Prefill runs in chunks of a fixed token budget (gouthm.com "The KV cache is
 *     not your bottleneck", section "The fix that mattered") and can start after
 *     a cached prefix (daviddominguez.dev, section "A prefix already in the cache
 *     can skip its prefill").
 *
 * Attention of query head h at position t:
 *     s_j = scale * <q_t[h], k_j[h / G]>,  j = 0..t (the token sees itself)
 *     o   = sum_j softmax(s)_j * v_j[h / G],   G = Hq / Hkv
 * arithmetic in fp32, inputs and outputs in the cache dtype.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or synchronises; it keeps no state between calls
 *     (beyond cached device properties and the built-in scratch array of
 *     kvc_decode_append_attention_noalloc) and is safe to call from several
 *     host threads.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns.
 *   - Host-side validation happens before any launch: on a negative status
 *     nothing was enqueued. Device-side contract violations (a block id outside
 *     [0, num_blocks), a slot outside the pool, a context longer than the block
 *     table) never touch memory out of bounds: the offending read or write is
 *     skipped (reads yield zero) and, if `err_flag` is non-NULL, a bit is OR-ed
 *     into that device int32 (KVC_DEVERR_*).
 *   - Alignment: q, k, v, out, k_new, v_new, the K / V pools and workspaces
 *     must be 16-byte aligned (the kernels move rows in 16-byte chunks, and
 *     every supported row is a multiple of 16 bytes); int32 arrays (block
 *     tables, lengths, offsets, ids, positions, err_flag) and the fp8 scale
 *     pools 4-byte; slot lists (int64) 8-byte. torch allocations and views at
 *     whole-row offsets satisfy this. A misaligned pointer is rejected with
 *     KVC_ERR_ALIGN, after every other rule, before any launch.
 *   - Cache layout, per layer and per K / V:
 *         [num_blocks][num_kv_heads][block_size = 16][head_dim]
 *     so one (block, kv-head) tile is contiguous (4 KiB for head_dim 128, bf16).
 *   - Supported: dtype fp32 (head_dim 16, 32, 64, 128) and bf16 (head_dim 32,
 *     64, 128); G = Hq / Hkv in {1, 2, 4, 8}; block_size 16.
 *   - Quantised cache (KVC_FP8): the pools hold OCP FP8 E4M3 codes and two
 *     more fp32 pools hold one scale per (block, kv head, token) row, laid out
 *     [num_blocks][num_kv_heads][16]. A row x of head_dim values is stored as
 *     scale = amax / 448 (amax = max |x|) and codes = E4M3(x * (448 / amax))
 *     rounded to nearest, ties to even, clamped at 448 (a row with amax below
 *     2^-100: scale 0, codes 0); its value is code * scale. The gouthm.com page ("The KV cache
 *     is not your bottleneck", sections "The setup" and "What the profile
 *     said") names quantising the cache for memory headroom at a small
 *     accuracy cost and gives no scheme; this one keeps each appended row
 *     independent of the rows after it. Queries, new K/V and outputs are bf16.
 *     Supported by kvc_kv_append, kvc_paged_decode_attention,
 *     kvc_decode_append_attention, the chunked-prefill calls (which write
 *     the chunk quantised and dequantise tiles to bf16 as they stage them)
 *     and kvc_mixed_step_attention, with head_dim 64 or 128.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVC_F32 = 0, KVC_BF16 = 1, KVC_FP8 = 2 } kvc_dtype;

enum {
  KVC_OK = 0,
  KVC_ERR_NULL = -1,        /* a required pointer is NULL */
  KVC_ERR_SHAPE = -2,       /* inconsistent sizes (Hq % Hkv, negative counts, ...) */
  KVC_ERR_DTYPE = -3,       /* unknown dtype */
  KVC_ERR_UNSUPPORTED = -4, /* head_dim / block_size / G outside the supported set */
  KVC_ERR_WORKSPACE = -5,   /* workspace missing or smaller than the size query */
  KVC_ERR_LAUNCH = -6,      /* the HIP runtime rejected a launch */
  KVC_ERR_NO_BLOCKS = -7,   /* prefix cache, scheduler: not enough free or reusable blocks */
  KVC_ERR_STATE = -8,       /* prefix cache: a block released or committed that the
                               caller does not hold, or out of range */
  KVC_ERR_NO_MEMORY = -9,   /* host memory ran out (prefix cache, scheduler) */
  KVC_ERR_ALIGN = -10,      /* a pointer is not aligned as the conventions below require */
  KVC_ERR_SCRATCH = -11     /* kvc_decode_append_attention_noalloc: the call needs more than
                               the library's built-in KVC_SCRATCH_BYTES of scratch */
};

/* Size of the per-device scratch array of kvc_decode_append_attention_noalloc. */
#define KVC_SCRATCH_BYTES ((size_t)16 << 20)

/* Bits OR-ed into cache->err_flag by kernels that skipped an invalid access. */
enum {
  KVC_DEVERR_BLOCK_ID = 1,  /* block table entry outside [0, num_blocks) */
  KVC_DEVERR_SLOT = 2,      /* slot outside [0, num_blocks * block_size) */
  KVC_DEVERR_CONTEXT = 4,   /* context needs more blocks than the table row has */
  KVC_DEVERR_QUEUE = 8      /* mixed-batch kernel: a wait for its first phase gave up (the
                               workspace header was not zero at the start of the call) */
};

/* One layer's paged cache. Pointers are device memory owned by the caller. */
typedef struct {
  void* k_cache;      /* [num_blocks][num_kv_heads][block_size][head_dim], dtype */
  void* v_cache;      /* same shape */
  int32_t num_blocks;
  int32_t block_size; /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;      /* kvc_dtype */
  int32_t* err_flag;  /* optional device int32 (may be NULL), see KVC_DEVERR_* */
  float* k_scale;     /* KVC_FP8 only: [num_blocks][num_kv_heads][16] fp32 row scales */
  float* v_scale;     /* (NULL for the other dtypes) */
} kvc_cache;

/* Host-only. Raw K+V bytes one token occupies across `layers` layers:
 * 2 * layers * kv_heads * head_dim * dtype_bytes (aiwithghost.com, section "How
 * KV cache memory limits concurrency"; daviddominguez.dev, section "What prefill
 * stores and decode reads"). Returns -1 on a negative argument. */
int64_t kvc_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                               int32_t dtype_bytes);

/* Slot of each new token: slot[t] = block_table[seq_ids[t]][p / bs] * bs + p % bs
 * with p = positions[t]; p < 0 gives slot -1 (a padding token). The cache is a
 * pool of fixed 16-token blocks that each sequence reaches through its own block
 * table (daviddominguez.dev "The KV cache and prefix caching", sections "What
 * prefill stores and decode reads" (PagedAttention) and "A prefix already in
 * the cache can skip its prefill" (16-token blocks)); the slot is where
 * position p of that sequence lives in the pool.
 *   block_table  device int32 [n_seqs][max_blocks] (row-major)
 *   seq_ids      device int32 [T], row of block_table for each token; a row
 *                outside [0, n_seqs) gives slot -1 and KVC_DEVERR_CONTEXT
 *   positions    device int32 [T], logical position of each token
 *   slot_mapping device int64 [T], written
 *   num_blocks   pool size, for the range check (bad ids give slot -1 + flag)
 *   err_flag     optional device int32
 * Block tables hold physical block ids in any order; the same ids are used by
 * every layer's pool. */
int kvc_slot_mapping(const int32_t* block_table, int32_t n_seqs, int32_t max_blocks,
                     int32_t num_blocks, const int32_t* seq_ids, const int32_t* positions, int32_t T,
                     int32_t block_size, int64_t* slot_mapping, int32_t* err_flag,
                     void* stream);

/* Append: k_cache[slot / bs][h][slot % bs][:] = k[t][h][:], same for v. Each
 * step stores the new position's key and value once, and later steps only read
 * them (aiwithghost.com "KV cache and continuous batching: 1,000 people ask AI",
 * section "What does a KV cache keep?"; daviddominguez.dev, section "What
 * prefill stores and decode reads").
 *   k, v          device [T][num_kv_heads][head_dim], cache dtype (no conversion:
 *                 the cache contents are bit-exact copies); bf16 for a KVC_FP8
 *                 cache, whose rows are quantised as the header describes
 *                 (codes into the pools, scales into k_scale / v_scale)
 *   slot_mapping  device int64 [T]; slot < 0 skips the token
 * T may be 0 (nothing is launched). */
int kvc_kv_append(const kvc_cache* cache, const int64_t* slot_mapping, const void* k,
                  const void* v, int32_t T, void* stream);

/* Bytes of scratch kvc_paged_decode_attention needs for these sizes (split-K
 * partial results). Depends only on its arguments. */
size_t kvc_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim,
                                  int32_t max_context_len);

/* Paged GQA decode attention for a batch of sequences of mixed lengths: each
 * sequence's newest query attends over every key and value its cache holds,
 * read through its block table, with Hq / Hkv query heads sharing each K/V head
 * (aiwithghost.com, section "What does a KV cache keep?"; daviddominguez.dev,
 * sections "What prefill stores and decode reads" and "The prompt is paid
 * once, the output is paid every step").
 *   q             device [B][Hq][head_dim], cache dtype (bf16 for KVC_FP8): each
 *                 sequence's newest query
 *   block_table   device int32 [B][max_blocks]
 *   context_lens  device int32 [B]: tokens in each sequence's cache INCLUDING the
 *                 newest one (append first, then attend). 0 gives a zero output.
 *   max_context_len  host-known upper bound of context_lens (sizes the grid;
 *                 no device-to-host copy is made)
 *   softmax_scale usually 1/sqrt(head_dim)
 *   out           device [B][Hq][head_dim], cache dtype (bf16 for KVC_FP8; bf16
 *                 outputs are rounded to nearest even)
 *   workspace     device scratch of >= kvc_decode_workspace_bytes(...) bytes, no
 *                 initialisation needed; may be NULL when max_context_len fits one
 *                 partition (the size query then returns 0).
 * Long contexts are split over several workgroups (split-K) whose partial
 * softmax states are merged by a second kernel on the same stream. */
int kvc_paged_decode_attention(const kvc_cache* cache, const void* q, int32_t B, int32_t Hq,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* context_lens, int32_t max_context_len,
                               float softmax_scale, void* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* One decode step in one launch: for every sequence b with context_lens[b] >= 1,
 * write k_new[b], v_new[b] ([num_kv_heads][head_dim], cache dtype; bf16 for
 * KVC_FP8, quantised on write) at position context_lens[b] - 1 through the
 * block table (append first), then attend q[b]
 * over positions 0 .. context_lens[b] - 1 (aiwithghost.com, section "What does a
 * KV cache keep?": compute the new token's K/V/Q, append, attend over everything
 * stored). Same arguments, outputs and workspace rule as
 * kvc_paged_decode_attention; the cache and `out` end up bit-identical to
 * kvc_slot_mapping + kvc_kv_append + kvc_paged_decode_attention. */
int kvc_decode_append_attention(const kvc_cache* cache, const void* q, const void* k_new,
                                const void* v_new, int32_t B, int32_t Hq,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* context_lens, int32_t max_context_len,
                                float softmax_scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* kvc_decode_append_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc) and so cannot provide a workspace: the split-K partial results go
 * to a scratch array inside the library instead, KVC_SCRATCH_BYTES (16 MiB) per
 * device, held from the first call on a device until the process ends. The
 * call allocates nothing; the caller still passes every input and output.
 * Arguments, outputs and results as kvc_decode_append_attention (same kernels,
 * same bits), without the workspace.
 *   Returns KVC_ERR_SCRATCH, before any launch, when the split-K partials
 *   would exceed KVC_SCRATCH_BYTES (B * Hq * partitions * (4 * head_dim + 8)
 *   bytes, partitions chosen as for kvc_decode_append_attention; C5's 8 x
 *   32,000-token decode needs about 1 MiB).
 * Every call on a device shares that device's array (no initialisation is
 * needed: each call writes the partials it reads), so calls that overlap on
 * one device, on different streams or from different host threads, race and
 * must be ordered by the caller. */
int kvc_decode_append_attention_noalloc(const kvc_cache* cache, const void* q, const void* k_new,
                                        const void* v_new, int32_t B, int32_t Hq,
                                        const int32_t* block_table, int32_t max_blocks,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        float softmax_scale, void* out, void* stream);

/* Chunked prefill: write a prompt chunk's K/V into the cache, then causal
 * attention of each chunk position over the cached prefix plus the chunk's
 * positions up to and including itself. Prompts run in chunks of a token
 * budget so decode rows wait at most one chunk (gouthm.com "The KV cache is not
 * your bottleneck", section "The fix that mattered"), a chunk can start after
 * a prefix already cached (daviddominguez.dev, section "A prefix already in
 * the cache can skip its prefill"), and the prompt's positions are processed
 * together as matrix products (aiwithghost.com, section "What does a KV cache
 * keep?").
 *   q             device [total_tokens][Hq][head_dim], chunks of all sequences
 *                 packed back to back
 *   k, v          device [total_tokens][num_kv_heads][head_dim]: the chunk's K/V
 *   cu_chunk_lens device int32 [n_seqs + 1]: chunk i is rows cu[i] .. cu[i+1]-1
 *   prefix_lens   device int32 [n_seqs]: tokens already cached before the chunk
 *                 (the chunk covers positions prefix .. prefix + C - 1)
 *   block_table   device int32 [n_seqs][max_blocks], covering prefix + chunk
 *   total_tokens, max_chunk_len  host-known: cu[n_seqs] and max_i C_i
 *   out           device [total_tokens][Hq][head_dim], cache dtype
 * The K/V write completes before the attention reads (same stream). */
int kvc_chunked_prefill_attention(const kvc_cache* cache, const void* q, const void* k,
                                  const void* v, int32_t n_seqs, const int32_t* cu_chunk_lens,
                                  const int32_t* prefix_lens, int32_t total_tokens,
                                  int32_t max_chunk_len, const int32_t* block_table,
                                  int32_t max_blocks, int32_t Hq, float softmax_scale,
                                  void* out, void* stream);

/* Bytes of workspace kvc_chunked_prefill_attention_split needs for these sizes
 * (0: no key-range split, no workspace). max_context_len bounds prefix + chunk
 * over the batch; num_kv_heads is the cache's. 0 for invalid sizes too. */
size_t kvc_prefill_workspace_bytes(int32_t n_seqs, int32_t total_tokens, int32_t max_chunk_len,
                                   int32_t max_context_len, int32_t Hq, int32_t num_kv_heads,
                                   int32_t head_dim);

/* kvc_chunked_prefill_attention for chunks too short to fill the GPU over a
 * long cached prefix (for example the tokens left after a prefix-cache hit,
 * daviddominguez.dev, section "A prefix already in the cache can skip its
 * prefill"): when the query tiles alone give too few workgroups, each one's
 * keys are split into ranges whose partial softmax states a second kernel
 * merges on the same stream (the log-sum-exp rule of the split decode).
 *   max_context_len  host-known bound on prefix + chunk over the batch; a
 *                    sequence past it sets KVC_DEVERR_CONTEXT (its rows are
 *                    then incomplete)
 *   workspace        device scratch of >= kvc_prefill_workspace_bytes(...)
 *                    bytes, 16-byte aligned, no initialisation needed; may be
 *                    NULL when that size is 0
 * Other arguments and outputs as kvc_chunked_prefill_attention; with no split
 * the two calls run the same kernel and give the same bits.
 * Returns KVC_ERR_WORKSPACE when the workspace is missing or too small. */
int kvc_chunked_prefill_attention_split(const kvc_cache* cache, const void* q, const void* k,
                                        const void* v, int32_t n_seqs,
                                        const int32_t* cu_chunk_lens, const int32_t* prefix_lens,
                                        int32_t total_tokens, int32_t max_chunk_len,
                                        int32_t max_context_len, const int32_t* block_table,
                                        int32_t max_blocks, int32_t Hq, float softmax_scale,
                                        void* out, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* One continuous-batching step in ONE launch: decode rows and prefill chunks
 * together (aiwithghost.com "KV cache and continuous batching: 1,000 people
 * ask AI", section "How does continuous batching share the server?": the batch
 * is rebuilt every step and newly admitted requests start with their prefill
 * next to rows that decode; gouthm.com "The KV cache is not your bottleneck",
 * section "The fix that mattered": decode rows plus prefill chunks under a
 * token budget). Computes what kvc_decode_append_attention (decode rows) and
 * kvc_chunked_prefill_attention (chunks) compute, in a persistent kernel whose
 * workgroups take work items from a device queue: first the chunks' K/V
 * writes (and, for a large decode batch, a longest-first order of the decode
 * rows), then prefill query tiles (later tiles first), then decode items (one
 * row and kv head each: the row's new K/V write, then attention over its whole
 * context).
 * Prefill rows equal kvc_chunked_prefill_attention's bit for bit; decode rows
 * are the same computation with a row's blocks spread over 8 waves of one
 * workgroup instead of split over workgroups (another summation order).
 * Fields: the arguments of those two calls; a part with count 0 may leave its
 * pointers NULL. Decode rows and prefill chunks must belong to different
 * sequences (their blocks may alias only where both only read, e.g. a shared
 * cached prefix). */
typedef struct {
  int32_t n_decode;                   /* decode rows, <= 4096 */
  const void* q_decode;               /* [n_decode][Hq][head_dim] */
  const void* k_new;                  /* [n_decode][num_kv_heads][head_dim], position ctx - 1 */
  const void* v_new;
  const int32_t* decode_block_table;  /* [n_decode][decode_max_blocks] */
  int32_t decode_max_blocks;
  const int32_t* decode_context_lens; /* [n_decode], counting the new token */
  int32_t decode_max_context;         /* host-known bound of decode_context_lens */
  void* out_decode;                   /* [n_decode][Hq][head_dim] */
  int32_t n_prefill;                  /* prefill chunks */
  const void* q_prefill;              /* [prefill_total_tokens][Hq][head_dim] */
  const void* k_prefill;              /* [prefill_total_tokens][num_kv_heads][head_dim] */
  const void* v_prefill;
  const int32_t* cu_chunk_lens;       /* [n_prefill + 1] */
  const int32_t* prefix_lens;         /* [n_prefill] */
  int32_t prefill_total_tokens;
  int32_t prefill_max_chunk;
  const int32_t* prefill_block_table; /* [n_prefill][prefill_max_blocks] */
  int32_t prefill_max_blocks;
  void* out_prefill;                  /* [prefill_total_tokens][Hq][head_dim] */
} kvc_mixed_batch;

/* Bytes of workspace kvc_mixed_step_attention needs: a 256-byte queue header
 * and the decode row order (256 + n_decode * 4, rounded up to 256). 0 for
 * invalid sizes. */
size_t kvc_mixed_workspace_bytes(int32_t n_decode, int32_t decode_max_context, int32_t Hq,
                                 int32_t num_kv_heads, int32_t head_dim);

/* Runs one mixed step (see kvc_mixed_batch) on `stream`.
 *   workspace  device memory of >= kvc_mixed_workspace_bytes(...) bytes, 16-byte
 *              aligned. Its first 256 bytes (the queue header) must be zero
 *              when a call starts: zero them once when the workspace is
 *              allocated; every call leaves them zero again. Calls that share
 *              a workspace must not overlap (same stream, or ordered).
 * Supported: bf16 and fp8 caches with head_dim 64 or 128 and fp32 caches with
 * head_dim 32, G = Hq / num_kv_heads in {1, 2, 4}; KVC_ERR_UNSUPPORTED
 * otherwise. With an fp8 cache the new decode rows and the chunks are written
 * quantised (the codes and scales kvc_kv_append and the chunked-prefill calls
 * write), and q, k_new, v_new, the chunks' K/V and the outputs are bf16.
 * Returns KVC_ERR_WORKSPACE for a missing or short workspace and validates
 * like the two calls it replaces.
 * Route: the two separate calls are the default. On MI355X this one launch
 * ties with them on a skewed 206-row decode batch with four 2,048-token
 * chunks over bf16 (0.97-1.03x), and loses over fp8 (4%), on the steps of a
 * 16-slot serving queue (20-27%) and on a uniform decode-only batch (8%):
 * its decode waves keep fewer blocks in flight (its prefill items set its
 * register budget).
 * Callers that want the faster route per step without measuring it
 * themselves can use the Python package's StepRunner, which takes the
 * separate calls for single-kind steps and times both routes on the first
 * steps of each size class of mixed steps. */
int kvc_mixed_step_attention(const kvc_cache* cache, const kvc_mixed_batch* batch, int32_t Hq,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Streaming-read probe, for measurement only: reads `bytes` bytes of device
 * memory at `data` once, front to back, with 128-bit non-temporal loads (the
 * plainest read pattern, so its rate over a buffer much larger than the
 * caches is the HBM read ceiling of the box the kernels above run on).
 *   data   device memory, 16-byte aligned; bytes a multiple of 16 (0 allowed)
 *   out    device uint32[kvc_stream_read_groups()]: workgroup g writes the
 *          wrapping 32-bit sum of the 32-bit words it read, so the sum of all
 *          entries (mod 2^32) is the sum of all words of the buffer
 * Async on `stream`; KVC_ERR_NULL / KVC_ERR_SHAPE / KVC_ERR_ALIGN before any
 * launch. */
int32_t kvc_stream_read_groups(void);
int kvc_stream_read(const void* data, size_t bytes, uint32_t* out, void* stream);

/* Static string for a status code. */
const char* kvc_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
