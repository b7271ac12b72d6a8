/*
 * kvc_prefix.h - prefix caching for the paged KV cache: a host-side block
 * manager that lets a prompt reuse the cached K/V of its opening blocks.
 *
 * What it does (restated from daviddominguez.dev "The KV cache and prefix
 * caching", section "A prefix already in the cache can skip its prefill"):
 *   - a prompt is hashed block by block and matched against blocks already
 *     held; prefill then starts after the matched part, over the matched
 *     blocks as its cached prefix (kvc_chunked_prefill_attention with
 *     prefix_len = block_size * matched);
 *   - block identifiers are chained: each covers its block's tokens and the
 *     identifier of the block before it, so a hit starts at position 0 and is
 *     a contiguous prefix (a prompt that differs at token 3 shares nothing);
 *   - hits are whole blocks of 16 tokens; the last partial block is recomputed;
 *     the match is on exact token ids (lookups compare the tokens, a hash only
 *     selects the candidates).
 *
 * Choices where the page is silent:
 *   - at least one token is always left to prefill, so at most
 *     (n_tokens - 1) / block_size blocks of a prompt match;
 *   - a block becomes matchable when committed (full blocks only, once their
 *     K/V are written); committing an identity that is already cached keeps
 *     the cached block, and the duplicate and the sequence's later blocks stay
 *     ordinary blocks (they would follow a block the sequence does not hold);
 *   - allocation takes the lowest-numbered free block, then reuses the least
 *     recently released unreferenced cached block (its identity is dropped);
 *     it is all or nothing;
 *   - a release drops one reference from each block, last block first, so a
 *     sequence's deeper blocks are reused before its opening ones.
 *
 * Block ids are indices into the pool's first dimension and are shared by all
 * layers, so one kvc_prefix_cache serves every layer's kvc_cache of one pool.
 * Shared blocks appear in several sequences' block tables; the decode and
 * prefill kernels read such aliased ids as they read any other.
 *
 * Host memory only: no call touches the GPU. An object is not thread-safe;
 * use it from one thread at a time. Errors return a negative kvc status
 * (kvc.h) and leave the object unchanged.
 */
#ifndef KVC_PREFIX_H
#define KVC_PREFIX_H

#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_prefix_cache kvc_prefix_cache;

/* A manager for a pool of num_blocks blocks (all free) of block_size tokens
 * (16). Returns NULL when num_blocks < 0, block_size != 16 or memory runs out. */
kvc_prefix_cache* kvc_prefix_cache_create(int32_t num_blocks, int32_t block_size);

/* Frees the manager (NULL is ignored). */
void kvc_prefix_cache_destroy(kvc_prefix_cache* pc);

/* Matches tokens[0 .. n_tokens) against the cached blocks. Writes the ids of
 * the longest cached whole-block prefix (at most max_blocks of them) to
 * block_ids and takes one reference on each. Returns the number of blocks
 * matched (>= 0; prefill starts at block_size times that), or KVC_ERR_NULL /
 * KVC_ERR_SHAPE. */
int32_t kvc_prefix_cache_match(kvc_prefix_cache* pc, const int32_t* tokens, int32_t n_tokens,
                               int32_t* block_ids, int32_t max_blocks);

/* Takes n blocks for new K/V, one reference each, ids written to block_ids.
 * Returns n, or KVC_ERR_NO_BLOCKS (nothing taken) when fewer than n blocks are
 * free or reusable. */
int32_t kvc_prefix_cache_allocate(kvc_prefix_cache* pc, int32_t n, int32_t* block_ids);

/* Makes the full blocks of a sequence matchable once their K/V are written:
 * block_ids[i] holds tokens[block_size * i .. block_size * (i + 1)) for every
 * full block i < n_blocks. The caller must hold a reference on each.
 * Returns KVC_OK, or KVC_ERR_STATE (nothing changed) when a block is not held,
 * out of range, or already cached under a different prefix. */
int32_t kvc_prefix_cache_commit(kvc_prefix_cache* pc, const int32_t* tokens, int32_t n_tokens,
                                const int32_t* block_ids, int32_t n_blocks);

/* Drops one reference from each of the n blocks (from the last to the first).
 * A block left with none becomes free, or, if it is cached, reusable.
 * Returns KVC_OK, or KVC_ERR_STATE (nothing changed) when some block would
 * drop more references than it holds. */
int32_t kvc_prefix_cache_release(kvc_prefix_cache* pc, const int32_t* block_ids, int32_t n);

/* References held on a block, or KVC_ERR_STATE for an id out of range. */
int32_t kvc_prefix_cache_refcount(const kvc_prefix_cache* pc, int32_t block_id);

/* Number of free blocks, of cached blocks (matchable, referenced or not) and of
 * referenced blocks. Any pointer may be NULL. Returns KVC_OK. */
int32_t kvc_prefix_cache_counts(const kvc_prefix_cache* pc, int32_t* n_free, int32_t* n_cached,
                                int32_t* n_referenced);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PREFIX_H */
