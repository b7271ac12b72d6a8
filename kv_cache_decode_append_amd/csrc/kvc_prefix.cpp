// Prefix caching: the host-side block manager behind include/kvc_prefix.h.
//
// A prompt reuses the cached K/V of its opening blocks (daviddominguez.dev "The
// KV cache and prefix caching", section "A prefix already in the cache can
// skip its prefill"). Block identities are chained: block i of a prompt is
// known by its own tokens together with the identity of block i-1, so a hit is
// a contiguous prefix from position 0. Lookups hash that chain (FNV-1a over the
// token ids, continued from the previous block's hash) to select candidates and
// then compare exactly: the candidate's tokens, and its parent, which must be
// the block matched one step earlier (by id and by the generation that id had
// when the child was registered, so an id reused for another prefix never
// carries a stale child along).

#include <stdint.h>

#include <iterator>
#include <list>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "kvc_prefix.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = parent;
  for (int i = 0; i < n; ++i) {
    uint32_t t = (uint32_t)tokens[i];
    for (int b = 0; b < 4; ++b) {
      h ^= (t >> (8 * b)) & 0xffu;
      h *= kFnvPrime;
    }
  }
  return h;
}

struct BlockInfo {
  bool cached = false;          // holds a matchable prefix
  uint64_t hash = 0;            // chain hash of the prefix it ends
  int32_t parent = -1;          // cached block of the previous prefix block, -1 for block 0
  uint32_t parent_gen = 0;      // that block's generation when this one was registered
  std::vector<int32_t> tokens;  // this block's tokens
  bool in_lru = false;
  std::list<int32_t>::iterator lru_it;
};

}  // namespace

struct kvc_prefix_cache {
  int32_t num_blocks = 0;
  int32_t bs = 16;
  std::vector<int32_t> ref;
  std::vector<uint32_t> gen;    // bumped whenever a block's cached identity is dropped
  std::vector<BlockInfo> info;
  std::set<int32_t> free_blocks;                      // lowest id first
  std::unordered_multimap<uint64_t, int32_t> table;  // chain hash -> cached block
  std::list<int32_t> lru;                             // unreferenced cached blocks, oldest first
  int32_t n_cached = 0;
  int32_t n_referenced = 0;

  // cached block holding (parent, tokens) under chain hash h, or -1
  int32_t find(uint64_t h, int32_t parent, const int32_t* tokens) const {
    auto range = table.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const BlockInfo& b = info[it->second];
      if (b.parent != parent) continue;
      if (parent >= 0 && b.parent_gen != gen[parent]) continue;
      bool same = true;
      for (int i = 0; i < bs && same; ++i) same = b.tokens[i] == tokens[i];
      if (same) return it->second;
    }
    return -1;
  }

  void drop_identity(int32_t blk) {
    BlockInfo& b = info[blk];
    auto range = table.equal_range(b.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == blk) {
        table.erase(it);
        break;
      }
    b.cached = false;
    b.tokens.clear();
    ++gen[blk];
    --n_cached;
  }

  void add_ref(int32_t blk) {
    if (ref[blk]++ == 0) {
      ++n_referenced;
      if (info[blk].in_lru) {
        lru.erase(info[blk].lru_it);
        info[blk].in_lru = false;
      }
    }
  }
};

extern "C" kvc_prefix_cache* kvc_prefix_cache_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 0 || block_size != 16) return nullptr;
  kvc_prefix_cache* pc = new (std::nothrow) kvc_prefix_cache();
  if (!pc) return nullptr;
  try {
    pc->num_blocks = num_blocks;
    pc->bs = block_size;
    pc->ref.assign(num_blocks, 0);
    pc->gen.assign(num_blocks, 0);
    pc->info.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) pc->free_blocks.insert(pc->free_blocks.end(), b);
  } catch (...) {
    delete pc;
    return nullptr;
  }
  return pc;
}

extern "C" void kvc_prefix_cache_destroy(kvc_prefix_cache* pc) { delete pc; }

extern "C" int32_t kvc_prefix_cache_match(kvc_prefix_cache* pc, const int32_t* tokens,
                                          int32_t n_tokens, int32_t* block_ids,
                                          int32_t max_blocks) {
  if (!pc) return KVC_ERR_NULL;
  if (n_tokens < 0 || max_blocks < 0) return KVC_ERR_SHAPE;
  const int32_t limit = n_tokens > 0 ? (n_tokens - 1) / pc->bs : 0;
  const int32_t want = limit < max_blocks ? limit : max_blocks;
  if (want > 0 && (!tokens || !block_ids)) return KVC_ERR_NULL;
  int32_t n = 0, parent = -1;
  uint64_t h = kFnvOffset;
  while (n < want) {
    const int32_t* blk_tokens = tokens + (size_t)n * pc->bs;
    h = chain_hash(h, blk_tokens, pc->bs);
    const int32_t blk = pc->find(h, parent, blk_tokens);
    if (blk < 0) break;
    block_ids[n++] = blk;
    parent = blk;
  }
  for (int32_t i = 0; i < n; ++i) pc->add_ref(block_ids[i]);
  return n;
}

extern "C" int32_t kvc_prefix_cache_allocate(kvc_prefix_cache* pc, int32_t n, int32_t* block_ids) {
  if (!pc) return KVC_ERR_NULL;
  if (n < 0) return KVC_ERR_SHAPE;
  if (n > 0 && !block_ids) return KVC_ERR_NULL;
  if ((size_t)n > pc->free_blocks.size() + pc->lru.size()) return KVC_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < n; ++i) {
    int32_t blk;
    if (!pc->free_blocks.empty()) {
      blk = *pc->free_blocks.begin();
      pc->free_blocks.erase(pc->free_blocks.begin());
    } else {
      blk = pc->lru.front();
      pc->lru.pop_front();
      pc->info[blk].in_lru = false;
      pc->drop_identity(blk);
    }
    pc->add_ref(blk);
    block_ids[i] = blk;
  }
  return n;
}

extern "C" int32_t kvc_prefix_cache_commit(kvc_prefix_cache* pc, const int32_t* tokens,
                                           int32_t n_tokens, const int32_t* block_ids,
                                           int32_t n_blocks) {
  if (!pc) return KVC_ERR_NULL;
  if (n_tokens < 0 || n_blocks < 0) return KVC_ERR_SHAPE;
  int32_t n = n_tokens / pc->bs;
  if (n_blocks < n) n = n_blocks;
  if (n > 0 && (!tokens || !block_ids)) return KVC_ERR_NULL;
  // validate first, so a rejected call changes nothing
  std::set<int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t blk = block_ids[i];
    if (blk < 0 || blk >= pc->num_blocks || pc->ref[blk] <= 0) return KVC_ERR_STATE;
    if (!seen.insert(blk).second) return KVC_ERR_STATE;
  }
  {
    // a block already cached must hold exactly this prefix; past the first
    // prefix that is not cached, no later one is, so a cached block there is
    // cached under another prefix
    int32_t parent = -1;
    uint64_t h = kFnvOffset;
    bool known = true;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t* blk_tokens = tokens + (size_t)i * pc->bs;
      const int32_t blk = block_ids[i];
      if (known) {
        h = chain_hash(h, blk_tokens, pc->bs);
        const int32_t have = pc->find(h, parent, blk_tokens);
        if (have >= 0) {
          if (pc->info[blk].cached && have != blk) return KVC_ERR_STATE;
          parent = have;
          continue;
        }
        known = false;
      }
      if (pc->info[blk].cached) return KVC_ERR_STATE;
    }
  }
  int32_t parent = -1;
  uint64_t h = kFnvOffset;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* blk_tokens = tokens + (size_t)i * pc->bs;
    h = chain_hash(h, blk_tokens, pc->bs);
    const int32_t blk = block_ids[i];
    const int32_t have = pc->find(h, parent, blk_tokens);
    if (have >= 0) {
      if (have != blk) break;  // a duplicate: later blocks would follow a block not held
      parent = have;
      continue;
    }
    BlockInfo& b = pc->info[blk];
    b.cached = true;
    b.hash = h;
    b.parent = parent;
    b.parent_gen = parent >= 0 ? pc->gen[parent] : 0;
    b.tokens.assign(blk_tokens, blk_tokens + pc->bs);
    pc->table.emplace(h, blk);
    ++pc->n_cached;
    parent = blk;
  }
  return KVC_OK;
}

extern "C" int32_t kvc_prefix_cache_release(kvc_prefix_cache* pc, const int32_t* block_ids,
                                            int32_t n) {
  if (!pc) return KVC_ERR_NULL;
  if (n < 0) return KVC_ERR_SHAPE;
  if (n > 0 && !block_ids) return KVC_ERR_NULL;
  std::unordered_map<int32_t, int32_t> drops;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t blk = block_ids[i];
    if (blk < 0 || blk >= pc->num_blocks) return KVC_ERR_STATE;
    if (++drops[blk] > pc->ref[blk]) return KVC_ERR_STATE;
  }
  for (int32_t i = n - 1; i >= 0; --i) {
    const int32_t blk = block_ids[i];
    if (--pc->ref[blk] > 0) continue;
    --pc->n_referenced;
    if (pc->info[blk].cached) {
      pc->lru.push_back(blk);
      pc->info[blk].lru_it = std::prev(pc->lru.end());
      pc->info[blk].in_lru = true;
    } else {
      pc->free_blocks.insert(blk);
    }
  }
  return KVC_OK;
}

extern "C" int32_t kvc_prefix_cache_refcount(const kvc_prefix_cache* pc, int32_t block_id) {
  if (!pc) return KVC_ERR_NULL;
  if (block_id < 0 || block_id >= pc->num_blocks) return KVC_ERR_STATE;
  return pc->ref[block_id];
}

extern "C" int32_t kvc_prefix_cache_counts(const kvc_prefix_cache* pc, int32_t* n_free,
                                           int32_t* n_cached, int32_t* n_referenced) {
  if (!pc) return KVC_ERR_NULL;
  if (n_free) *n_free = (int32_t)pc->free_blocks.size();
  if (n_cached) *n_cached = pc->n_cached;
  if (n_referenced) *n_referenced = pc->n_referenced;
  return KVC_OK;
}
