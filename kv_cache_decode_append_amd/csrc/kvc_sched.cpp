// Iteration-level scheduler and step builder behind include/kvc_sched.h.
//
// Each call to kvc_sched_next_step admits queued requests, picks the step's
// decode rows and prompt chunks under the policy (continuous batching with
// prefill-first or decode-first steps, or static groups; aiwithghost.com "KV
// cache and continuous batching: 1,000 people ask AI", section "How does
// continuous batching share the server?", and gouthm.com "The KV cache is not
// your bottleneck", section "The fix that mattered"), gives the step's rows the
// cache blocks their new tokens need, and writes the kernels' batch
// descriptors. Everything is planned on the side first, so a step the block
// pool cannot cover changes nothing.

#include <stdint.h>

#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "kvc_sched.h"

namespace {

constexpr int32_t kBlock = 16;

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + kBlock - 1) / kBlock); }

struct Request {
  int32_t prompt = 0;
  int32_t answer = 0;
  int32_t covered = 0;    // prompt tokens prefilled
  int32_t generated = 0;  // answer tokens made
  std::vector<int32_t> blocks;
  bool prefilled() const { return covered == prompt; }
  bool done() const { return prefilled() && generated == answer; }
};

struct Chunk {
  int32_t id, start, take;
};

}  // namespace

struct kvc_sched {
  int32_t policy = 0;
  int32_t slots = 1;
  int32_t budget = 1;
  int32_t num_blocks = 0;
  int32_t max_blocks = 1;
  std::vector<Request> reqs;
  std::deque<int32_t> queue;
  std::vector<int32_t> running;  // admission order; static groups keep finished members
  // free pool: a flag per block, the count, and a bound below which no block
  // is free, so the lowest free id is found by scanning up from it
  std::vector<char> is_free;
  int32_t n_free = 0;
  int32_t lowest = 0;
  int32_t unfinished = 0;

  int32_t take_lowest() {
    while (!is_free[lowest]) ++lowest;
    is_free[lowest] = 0;
    --n_free;
    return lowest;
  }
  void give_back(int32_t b) {
    is_free[b] = 1;
    ++n_free;
    lowest = std::min(lowest, b);
  }
};

extern "C" kvc_sched* kvc_sched_create(int32_t policy, int32_t slots, int32_t token_budget,
                                       int32_t num_blocks, int32_t max_blocks_per_seq) {
  if (policy != KVC_SCHED_PREFILL_FIRST && policy != KVC_SCHED_DECODE_FIRST &&
      policy != KVC_SCHED_STATIC)
    return nullptr;
  if (slots < 1 || token_budget < 1 || num_blocks < 0 || max_blocks_per_seq < 1) return nullptr;
  kvc_sched* s = new (std::nothrow) kvc_sched();
  if (!s) return nullptr;
  try {
    s->policy = policy;
    s->slots = slots;
    s->budget = token_budget;
    s->num_blocks = num_blocks;
    s->max_blocks = max_blocks_per_seq;
    s->is_free.assign((size_t)num_blocks, 1);
    s->n_free = num_blocks;
  } catch (...) {
    delete s;
    return nullptr;
  }
  return s;
}

extern "C" void kvc_sched_destroy(kvc_sched* s) { delete s; }

extern "C" int32_t kvc_sched_submit(kvc_sched* s, int32_t prompt_len, int32_t answer_len) {
  if (!s) return KVC_ERR_NULL;
  if (prompt_len < 1 || answer_len < 1) return KVC_ERR_SHAPE;
  if (blocks_for((int64_t)prompt_len + answer_len - 1) > s->max_blocks) return KVC_ERR_SHAPE;
  if (s->reqs.size() >= (size_t)INT32_MAX) return KVC_ERR_SHAPE;
  const int32_t id = (int32_t)s->reqs.size();
  try {
    Request r;
    r.prompt = prompt_len;
    r.answer = answer_len;
    s->reqs.push_back(r);
    s->queue.push_back(id);
  } catch (...) {
    if (s->reqs.size() > (size_t)id) s->reqs.pop_back();
    return KVC_ERR_NO_MEMORY;
  }
  ++s->unfinished;
  return id;
}

extern "C" int32_t kvc_sched_unfinished(const kvc_sched* s) {
  return s ? s->unfinished : KVC_ERR_NULL;
}

extern "C" int32_t kvc_sched_next_step(kvc_sched* s, kvc_step* st) {
  if (!s || !st) return KVC_ERR_NULL;
  if (!st->decode_ids || !st->decode_context_lens || !st->decode_block_table ||
      !st->prefill_ids || !st->prefill_prefix_lens || !st->prefill_cu_chunk_lens ||
      !st->prefill_block_table || !st->first_token_ids || !st->finished_ids)
    return KVC_ERR_NULL;
  st->n_decode = st->n_prefill = st->n_first = st->n_finished = 0;
  st->decode_max_context = st->prefill_total_tokens = st->prefill_max_chunk = 0;
  st->prefill_max_context = 0;
  st->prefill_cu_chunk_lens[0] = 0;

  // admission, planned on a copy of the running list
  std::vector<int32_t> running = s->running;
  size_t admitted = 0;
  const bool group_start = s->policy == KVC_SCHED_STATIC && running.empty();
  if (s->policy != KVC_SCHED_STATIC || group_start)
    while (admitted < s->queue.size() && running.size() < (size_t)s->slots)
      running.push_back(s->queue[admitted++]);
  if (running.empty()) return 0;

  // the step's rows
  std::vector<int32_t> decode;
  std::vector<Chunk> chunks;
  std::vector<int32_t> pending, ready;
  for (int32_t r : running) {
    const Request& q = s->reqs[r];
    if (!q.prefilled())
      pending.push_back(r);
    else if (q.generated < q.answer)
      ready.push_back(r);
  }
  if (s->policy == KVC_SCHED_STATIC) {
    if (group_start)
      for (int32_t r : pending) chunks.push_back({r, 0, s->reqs[r].prompt});
    else
      decode = ready;
  } else {
    const bool decode_first = s->policy == KVC_SCHED_DECODE_FIRST;
    if (decode_first || pending.empty()) decode = ready;
    if (decode_first || !pending.empty()) {
      int32_t left = s->budget;
      for (int32_t r : pending) {
        if (left == 0) break;
        const Request& q = s->reqs[r];
        const int32_t take = std::min(q.prompt - q.covered, left);
        chunks.push_back({r, q.covered, take});
        left -= take;
      }
    }
  }

  // blocks: count first, so a pool that cannot cover the step changes nothing
  size_t need = 0;
  for (int32_t r : decode) {
    const Request& q = s->reqs[r];
    need += (size_t)std::max(0, blocks_for((int64_t)q.prompt + q.generated) - (int32_t)q.blocks.size());
  }
  for (const Chunk& c : chunks)
    need += (size_t)std::max(
        0, blocks_for((int64_t)c.start + c.take) - (int32_t)s->reqs[c.id].blocks.size());
  if (need > (size_t)s->n_free) return KVC_ERR_NO_BLOCKS;

  // room for everything the commit below stores, so it cannot fail halfway
  std::vector<char> active;
  try {
    active.assign(s->reqs.size(), 0);
    for (int32_t r : decode) {
      Request& q = s->reqs[r];
      q.blocks.reserve((size_t)blocks_for((int64_t)q.prompt + q.generated));
    }
    for (const Chunk& c : chunks)
      s->reqs[c.id].blocks.reserve((size_t)blocks_for((int64_t)c.start + c.take));
  } catch (...) {
    return KVC_ERR_NO_MEMORY;
  }

  // commit: admission, allocation, descriptors, then the step's effects
  {
    s->running.swap(running);
    s->queue.erase(s->queue.begin(), s->queue.begin() + (ptrdiff_t)admitted);
    auto grow = [&](Request& q, int64_t tokens) {
      const int32_t want = blocks_for(tokens);
      while ((int32_t)q.blocks.size() < want) q.blocks.push_back(s->take_lowest());
    };
    auto write_row = [&](int32_t* table, int32_t row, const Request& q) {
      int32_t* dst = table + (size_t)row * s->max_blocks;
      std::fill(dst, dst + s->max_blocks, -1);
      std::copy(q.blocks.begin(), q.blocks.end(), dst);
    };
    for (int32_t r : decode) {
      Request& q = s->reqs[r];
      const int32_t ctx = q.prompt + q.generated;
      grow(q, ctx);
      const int32_t i = st->n_decode++;
      st->decode_ids[i] = r;
      st->decode_context_lens[i] = ctx;
      write_row(st->decode_block_table, i, q);
      st->decode_max_context = std::max(st->decode_max_context, ctx);
    }
    for (const Chunk& c : chunks) {
      Request& q = s->reqs[c.id];
      grow(q, (int64_t)c.start + c.take);
      const int32_t i = st->n_prefill++;
      st->prefill_ids[i] = c.id;
      st->prefill_prefix_lens[i] = c.start;
      st->prefill_cu_chunk_lens[i + 1] = st->prefill_cu_chunk_lens[i] + c.take;
      write_row(st->prefill_block_table, i, q);
      st->prefill_max_chunk = std::max(st->prefill_max_chunk, c.take);
      st->prefill_max_context = std::max(st->prefill_max_context, c.start + c.take);
    }
    st->prefill_total_tokens = st->prefill_cu_chunk_lens[st->n_prefill];
  }

  for (const Chunk& c : chunks) {
    Request& q = s->reqs[c.id];
    q.covered += c.take;
    if (q.prefilled()) {
      q.generated = 1;
      st->first_token_ids[st->n_first++] = c.id;
    }
  }
  for (int32_t r : decode) ++s->reqs[r].generated;

  // leaving: in admission order, among the rows this step ran
  for (int32_t r : decode) active[r] = 1;
  for (const Chunk& c : chunks) active[c.id] = 1;
  for (int32_t r : s->running) {
    Request& q = s->reqs[r];
    if (!active[r] || !q.done()) continue;
    st->finished_ids[st->n_finished++] = r;
    for (int32_t b : q.blocks) s->give_back(b);
    q.blocks.clear();
    --s->unfinished;
  }
  if (s->policy == KVC_SCHED_STATIC) {
    bool all_done = true;
    for (int32_t r : s->running) all_done = all_done && s->reqs[r].done();
    if (all_done) s->running.clear();
  } else {
    s->running.erase(std::remove_if(s->running.begin(), s->running.end(),
                                    [&](int32_t r) { return s->reqs[r].done(); }),
                     s->running.end());
  }
  return 1;
}
