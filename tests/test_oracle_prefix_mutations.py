"""Planted mistakes in copies of oracle.prefix (CPU only): each must fail at
least one of the pins in tests/test_oracle_prefix.py."""
import pytest

from oracle.prefix import PrefixCache
from tests.test_oracle_prefix import PINS


class NoOneTokenCap(PrefixCache):
    def max_match_blocks(self, n_tokens):
        return n_tokens // self.bs


class PartialLastBlock(PrefixCache):
    def max_match_blocks(self, n_tokens):
        return max(0, (n_tokens + self.bs - 2) // self.bs)


class BlockLocalMatch(PrefixCache):
    """Compares each block's own tokens only, not the chain before it."""
    def match(self, tokens):
        tokens = list(tokens)
        by_block = {k[-self.bs:]: b for k, b in self.cached.items()}
        out = []
        for i in range(self.max_match_blocks(len(tokens))):
            blk = by_block.get(tuple(tokens[self.bs * i: self.bs * (i + 1)]))
            if blk is None:
                break
            out.append(blk)
        for blk in out:
            if self.ref[blk] == 0:
                self.lru.remove(blk)
            self.ref[blk] += 1
        return out


class ForwardRelease(PrefixCache):
    def release(self, block_ids):
        for blk in list(block_ids):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                (self.lru.append if blk in self.key_of else self.free.add)(blk)


class CommitOverwrites(PrefixCache):
    def commit(self, tokens, block_ids):
        tokens = list(tokens)
        for i in range(min(len(tokens) // self.bs, len(block_ids))):
            key = tuple(tokens[: self.bs * (i + 1)])
            old = self.cached.get(key)
            if old is not None:
                del self.key_of[old]
            self.cached[key] = block_ids[i]
            self.key_of[block_ids[i]] = key


MUTANTS = [NoOneTokenCap, PartialLastBlock, BlockLocalMatch, ForwardRelease, CommitOverwrites]


def _passes_all(cls):
    for pin in PINS:
        try:
            pin(cls)
        except Exception:
            return False
    return True


def test_oracle_passes_every_pin():
    assert _passes_all(PrefixCache)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_mutant_fails_a_pin(mutant):
    assert not _passes_all(mutant)
