"""The native prefix-cache block manager (include/kvc_prefix.h, host code, no
GPU) against the oracle: the page's worked rules, and identical results --
block ids, reference counts, counts, rejections -- over random operation
sequences."""
import json
import os
import random

import pytest

from oracle.prefix import PrefixCache as Oracle
from tests.test_oracle_prefix import GOLDEN, build_prompt

kvc = pytest.importorskip("kv_cache_decode_append_amd")


def test_golden_rules_through_the_library():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        pc = kvc.PrefixCache(1000)
        cached = list(range(case["cached_len"]))
        blocks = pc.allocate((len(cached) + 15) // 16)
        pc.commit(cached, blocks)
        prompt = build_prompt(cached, case["prompt"])
        got = pc.match(prompt)
        assert len(got) == case["expect_blocks"], case["name"]
        assert got == blocks[: len(got)], case["name"]
        assert len(prompt) - 16 * len(got) == case["expect_prefill_tokens"], case["name"]


def _same_state(lib, orc):
    f, c, r = lib.counts()
    assert (f, c, r) == (orc.n_free(), orc.n_cached(), orc.n_referenced())
    assert [lib.refcount(b) for b in range(lib.num_blocks)] == orc.ref


@pytest.mark.parametrize("seed,pool,alphabet", [(1, 64, 3), (2, 40, 2), (3, 200, 5), (4, 16, 2)])
def test_random_operations_match_the_oracle(seed, pool, alphabet):
    rng = random.Random(seed)
    lib, orc = kvc.PrefixCache(pool), Oracle(pool)
    live = []
    for step in range(2500):
        op = rng.random()
        if op < 0.5 or not live:
            # prompts share openings often: a few stems plus random tails
            stem = [(i * 7 + seed) % alphabet for i in range(rng.choice([0, 16, 33, 64, 100]))]
            p = stem + [rng.randrange(alphabet) for _ in range(rng.randrange(1, 70))]
            held_l, held_o = lib.match(p), orc.match(p)
            assert held_l == held_o, step
            need = (len(p) + 15) // 16 - len(held_l)
            fresh_l, fresh_o = lib.allocate(need), orc.allocate(need)
            assert fresh_l == fresh_o, step
            if fresh_l is None:
                lib.release(held_l)
                orc.release(held_o)
            else:
                blocks = held_l + fresh_l
                if rng.random() < 0.9:               # most sequences finish their prefill
                    lib.commit(p, blocks)
                    orc.commit(p, blocks)
                live.append(blocks)
        elif op < 0.9:
            blocks = live.pop(rng.randrange(len(live)))
            lib.release(blocks)
            orc.release(blocks)
        else:
            # a sequence grows by decode tokens and commits its new full block
            i = rng.randrange(len(live))
            more = lib.allocate(1)
            assert more == orc.allocate(1)
            if more is not None:
                live[i] = live[i] + more
        _same_state(lib, orc)


def test_rejections_change_nothing():
    lib = kvc.PrefixCache(8)
    a = list(range(48))
    blocks = lib.allocate(3)
    lib.commit(a, blocks)
    before = (lib.counts(), [lib.refcount(b) for b in range(8)])
    with pytest.raises(kvc.KvcError):
        lib.release([blocks[0], blocks[0]])          # one reference, dropped twice
    with pytest.raises(kvc.KvcError):
        lib.commit(a, [blocks[0], 7, blocks[2]])     # block 7 is not held
    with pytest.raises(kvc.KvcError):
        lib.commit(list(range(100, 148)), blocks)    # blocks cached under another prefix
    with pytest.raises(kvc.KvcError):
        lib.refcount(8)
    assert lib.allocate(6) is None                   # only 5 left
    assert (lib.counts(), [lib.refcount(b) for b in range(8)]) == before
    assert kvc.LIB.kvc_prefix_cache_create(-1, 16) is None
    assert kvc.LIB.kvc_prefix_cache_create(8, 32) is None


def test_large_pool_long_prompts():
    """A 2,000-token system prompt shared by 64 requests with distinct tails."""
    lib = kvc.PrefixCache(9200)
    system = [(i * 2654435761) % 128000 for i in range(1800)]
    first = system + [1] * 200
    b0 = lib.allocate(125)
    lib.commit(first, b0)
    for r in range(64):
        p = system + [(r * 997 + j) % 128000 for j in range(200 + r)]
        m = lib.match(p)
        assert m == b0[:112]
        fresh = lib.allocate((len(p) + 15) // 16 - 112)
        lib.commit(p, m + fresh)
    assert lib.refcount(b0[0]) == 65 and lib.refcount(b0[112]) == 1
