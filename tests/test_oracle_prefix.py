"""Pins for oracle.prefix: the page's prefix-caching rules as worked cases, a
brute-force definition of the match, and bookkeeping invariants."""
import json
import os
import random

import pytest

from oracle.prefix import PrefixCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prefix_rules.json")


def build_prompt(cached, spec):
    p = list(cached[: spec["keep"]])
    for i in spec.get("change_at", []):
        p[i] += 1_000_000
    p += [2_000_000 + i for i in range(spec.get("new_tail", 0))]
    return p


def pin_golden_rules(cls=PrefixCache):
    g = json.load(open(GOLDEN))
    assert g["block_size"] == 16
    for case in g["cases"]:
        pc = cls(1000)
        cached = list(range(case["cached_len"]))
        blocks = pc.allocate((len(cached) + 15) // 16)
        pc.commit(cached, blocks)
        prompt = build_prompt(cached, case["prompt"])
        got = pc.match(prompt)
        assert len(got) == case["expect_blocks"], case["name"]
        assert got == blocks[: len(got)], case["name"]
        start = 16 * len(got)
        assert start == case["expect_prefill_start"], case["name"]
        assert len(prompt) - start == case["expect_prefill_tokens"], case["name"]


def pin_cold_cache_matches_nothing(cls=PrefixCache):
    pc = cls(10)
    assert pc.match(list(range(100))) == []


def pin_partial_blocks_are_never_matchable(cls=PrefixCache):
    pc = cls(10)
    toks = list(range(40))                       # 2 full blocks + 8 tokens
    blocks = pc.allocate(3)
    pc.commit(toks, blocks)
    assert pc.n_cached() == 2
    assert pc.match(toks + [7] * 30) == blocks[:2]


def _lcp_blocks(a, b, bs):
    n = 0
    while n + bs <= min(len(a), len(b)) and a[n:n + bs] == b[n:n + bs] and a[:n] == b[:n]:
        n += bs
    return n // bs


def pin_brute_force_longest_whole_block_prefix(cls=PrefixCache):
    rng = random.Random(5)
    for trial in range(30):
        pc = cls(4000)
        base = [rng.randrange(50) for _ in range(300)]
        committed = []
        for _ in range(6):
            cut = rng.randrange(0, 300)
            p = base[:cut] + [rng.randrange(50) for _ in range(rng.randrange(0, 120))]
            held = pc.match(p)
            fresh = pc.allocate((len(p) + 15) // 16 - len(held))
            pc.commit(p, held + fresh)
            committed.append(p)
        for _ in range(10):
            cut = rng.randrange(0, 400)
            q = (base + [1] * 100)[:cut] + [rng.randrange(50) for _ in range(rng.randrange(0, 50))]
            expect = max([0] + [_lcp_blocks(q, c, 16) for c in committed if len(c) >= 16])
            # only whole blocks of committed prompts are cached; one token stays to prefill
            expect = min(expect, max(0, (len(q) - 1) // 16))
            got = pc.match(q)
            assert len(got) == expect, (trial, cut)
            pc.release(got)


def _check_states(pc):
    refd = {b for b, r in enumerate(pc.ref) if r > 0}
    lru = set(pc.lru)
    assert len(lru) == len(pc.lru)
    assert not (refd & pc.free) and not (refd & lru) and not (lru & pc.free)
    assert refd | lru | pc.free == set(range(len(pc.ref)))
    assert lru <= set(pc.key_of)
    assert set(pc.cached.values()) == set(pc.key_of)
    assert all(pc.cached[k] == b for b, k in pc.key_of.items())


def pin_random_operations_keep_states_consistent(cls=PrefixCache):
    rng = random.Random(11)
    pc = cls(64)
    live = []
    for step in range(3000):
        op = rng.random()
        if op < 0.45 or not live:
            p = [rng.randrange(4) for _ in range(rng.randrange(1, 100))]
            held = pc.match(p)
            need = (len(p) + 15) // 16 - len(held)
            fresh = pc.allocate(need)
            if fresh is None:
                pc.release(held)
                continue
            blocks = held + fresh
            pc.commit(p, blocks)
            live.append(blocks)
        else:
            pc.release(live.pop(rng.randrange(len(live))))
        _check_states(pc)
        held_counts = {}
        for blocks in live:
            for b in blocks:
                held_counts[b] = held_counts.get(b, 0) + 1
        assert all(pc.ref[b] == held_counts.get(b, 0) for b in range(64))


def pin_reuse_order_deeper_blocks_first(cls=PrefixCache):
    pc = cls(4)
    a = list(range(64))                          # 4 full blocks
    blocks = pc.allocate(4)
    pc.commit(a, blocks)
    pc.release(blocks)                           # last block released first
    assert pc.lru == blocks[::-1]
    got = pc.allocate(1)                         # nothing free: reuse the deepest block
    assert got == [blocks[3]]
    assert len(pc.match(a + [9])) == 3           # its identity is gone, the prefix stays
    with pytest.raises(ValueError):
        pc.release([got[0], got[0]])


def pin_commit_keeps_the_first_copy(cls=PrefixCache):
    pc = cls(8)
    a = list(range(32))
    b1 = pc.allocate(2)
    b2 = pc.allocate(2)                          # the same prompt computed cold twice
    pc.commit(a, b1)
    pc.commit(a, b2)
    assert pc.n_cached() == 2 and set(pc.key_of) == set(b1)
    pc.release(b2)
    assert set(b2) <= pc.free
    # a sequence computed cold over the same opening: its duplicate first block
    # stops registration, so its third block does not become matchable
    c = a + list(range(100, 116))
    b3 = pc.allocate(3)
    pc.commit(c, b3)
    assert pc.n_cached() == 2
    assert len(pc.match(c + [0])) == 2


def pin_no_mixing_of_cached_prompts(cls=PrefixCache):
    """Block identities are chained: the first block of one cached prompt and
    the second block of another do not combine into a hit."""
    pc = cls(16)
    x = [1] * 16 + [2] * 16 + [0]
    y = [3] * 16 + [4] * 16 + [0]
    pc.commit(x, pc.allocate(3))
    pc.commit(y, pc.allocate(3))
    assert len(pc.match([1] * 16 + [4] * 16 + [5])) == 1
    assert len(pc.match(y)) == 2


PINS = [pin_golden_rules, pin_no_mixing_of_cached_prompts, pin_cold_cache_matches_nothing, pin_partial_blocks_are_never_matchable,
        pin_brute_force_longest_whole_block_prefix, pin_random_operations_keep_states_consistent,
        pin_reuse_order_deeper_blocks_first, pin_commit_keeps_the_first_copy]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
