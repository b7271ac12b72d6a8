"""Prefix caching: reuse of the cached K/V of a prompt's opening blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (daviddominguez page "The KV cache and prefix caching",
section "A prefix already in the cache can skip its prefill"):

* a prompt is matched block by block against blocks the server already holds,
  and prefill starts after the matched part;
* a hit starts at position 0 and is a contiguous prefix: a block can match only
  if every token up to and including it equals a cached sequence's, because a
  position's key and value depend on every earlier position (a prompt that
  differs at token 3 shares nothing);
* hits are counted in whole blocks of 16 tokens, so the last partial block is
  recomputed; the match is on exact token ids.

The pages describe chained block identifiers: each covers the block's tokens
and the identifier of the block before it. The plain form of that identity,
used here, is the whole token prefix a block ends: block i of a prompt is
known by ``tuple(tokens[:16 * (i + 1)])``.

Readings (the pages are silent):

* at least one token is always left to prefill (its query produces the next
  token), so at most ``(n - 1) // 16`` blocks of an n-token prompt match;
* a block becomes matchable when its sequence commits it: only full blocks,
  after their K/V have been written;
* committing a block whose identity is already cached keeps the cached block;
  the duplicate stays unregistered and is freed when released, and the
  sequence's later blocks are not registered either (they would follow a block
  the sequence does not hold);
* allocation takes the lowest-numbered free block; when none is free it reuses
  the least recently released unreferenced cached block, whose identity is
  dropped; allocation is all or nothing;
* a release drops one reference from each block of a sequence, from its last
  block to its first, so deeper blocks are reused before their prefixes.

Pins (tests/test_oracle_prefix.py): the page's rules as worked cases
(tests/golden/prefix_rules.json), brute force over the committed prompts, and
bookkeeping invariants under random operation sequences.
"""
from __future__ import annotations


class PrefixCache:
    """Block pool with reference counts and prefix matching, one Python step per block."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool shape")
        self.bs = block_size
        self.ref = [0] * num_blocks
        self.free = set(range(num_blocks))
        self.cached = {}            # token prefix (tuple) -> block id
        self.key_of = {}            # block id -> token prefix it ends
        self.lru = []               # unreferenced cached blocks, least recently released first

    # -- queries -----------------------------------------------------------
    def max_match_blocks(self, n_tokens: int) -> int:
        return max(0, (n_tokens - 1) // self.bs)

    def n_free(self) -> int:
        return len(self.free)

    def n_cached(self) -> int:
        return len(self.key_of)

    def n_referenced(self) -> int:
        return sum(1 for r in self.ref if r > 0)

    # -- operations --------------------------------------------------------
    def match(self, tokens) -> list:
        """Blocks holding the longest cached whole-block prefix of ``tokens``;
        takes one reference on each."""
        tokens = list(tokens)
        out = []
        for i in range(self.max_match_blocks(len(tokens))):
            blk = self.cached.get(tuple(tokens[: self.bs * (i + 1)]))
            if blk is None:
                break
            out.append(blk)
        for blk in out:
            if self.ref[blk] == 0:
                self.lru.remove(blk)
            self.ref[blk] += 1
        return out

    def allocate(self, n: int):
        """``n`` fresh blocks with one reference each, or None (nothing taken)."""
        if n < 0:
            raise ValueError("negative count")
        if n > len(self.free) + len(self.lru):
            return None
        out = []
        for _ in range(n):
            if self.free:
                blk = min(self.free)
                self.free.remove(blk)
            else:
                blk = self.lru.pop(0)
                del self.cached[self.key_of.pop(blk)]
            self.ref[blk] = 1
            out.append(blk)
        return out

    def commit(self, tokens, block_ids) -> None:
        """Make the full blocks of a sequence matchable (their K/V are written).

        Registration follows the sequence's own chain: at the first block whose
        prefix is already cached in another block (a duplicate computed cold),
        it stops, so no registered block ever follows a block its sequence
        does not hold."""
        tokens = list(tokens)
        n = min(len(tokens) // self.bs, len(block_ids))
        if len(set(block_ids[:n])) < n:
            raise ValueError("a block listed twice")
        for i in range(n):
            blk = block_ids[i]
            if self.ref[blk] <= 0:
                raise ValueError("committing a block the sequence does not hold")
            key = tuple(tokens[: self.bs * (i + 1)])
            if blk in self.key_of and self.key_of[blk] != key:
                raise ValueError("block already cached under another prefix")
        for i in range(n):
            blk = block_ids[i]
            key = tuple(tokens[: self.bs * (i + 1)])
            if key in self.cached:
                if self.cached[key] != blk:
                    return
                continue
            self.cached[key] = blk
            self.key_of[blk] = key

    def release(self, block_ids) -> None:
        """Drop one reference from each block, last block first."""
        drops = {}
        for blk in block_ids:
            drops[blk] = drops.get(blk, 0) + 1
        for blk, n in drops.items():
            if self.ref[blk] < n:
                raise ValueError("releasing more references than a block holds")
        for blk in reversed(list(block_ids)):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                if blk in self.key_of:
                    self.lru.append(blk)
                else:
                    self.free.add(blk)
