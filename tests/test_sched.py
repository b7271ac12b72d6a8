"""The native scheduler and step builder (include/kvc_sched.h) against the
oracle scheduler: the same plans and the same batch descriptors, bit for bit,
on random queues; and its error paths. Host code only, no GPU."""
import random

import numpy as np
import pytest

from oracle import sched as OS

kvc = pytest.importorskip("kv_cache_decode_append_amd")

POLICIES = {"prefill_first": (kvc.SCHED_PREFILL_FIRST, OS.PREFILL_FIRST),
            "decode_first": (kvc.SCHED_DECODE_FIRST, OS.DECODE_FIRST),
            "static": (kvc.SCHED_STATIC, None)}


def _native_steps(policy, prompts, answers, slots, budget, num_blocks, max_blocks):
    s = kvc.Scheduler(policy, slots, budget, num_blocks, max_blocks)
    assert [s.submit(p, a) for p, a in zip(prompts, answers)] == list(range(len(prompts)))
    out = []
    while True:
        st = s.next_step()
        if st is None:
            break
        out.append(st)
        assert len(out) < 100000
    assert s.unfinished() == 0
    return out


def _oracle_steps(name, prompts, answers, slots, budget):
    if name == "static":
        return OS.static(prompts, answers, slots)
    return OS.continuous(prompts, answers, slots, budget, POLICIES[name][1])


def _compare(name, prompts, answers, slots, budget, num_blocks, max_blocks):
    want = _oracle_steps(name, prompts, answers, slots, budget)
    want_b = OS.step_batches(want, prompts, answers, num_blocks)
    got = _native_steps(POLICIES[name][0], prompts, answers, slots, budget, num_blocks, max_blocks)
    assert len(got) == len(want)
    for i, (g, w, wb) in enumerate(zip(got, want, want_b)):
        assert g.decode_ids.tolist() == w.decode, i
        assert [(int(r), int(s0), int(t)) for r, s0, t in zip(
            g.prefill_ids, g.prefill_prefix_lens, np.diff(g.prefill_cu_chunk_lens))] == w.prefill, i
        assert g.first_token_ids.tolist() == w.first_token, i
        assert g.finished_ids.tolist() == w.finished, i
        assert g.decode_context_lens.tolist() == [c for _, c, _ in wb["decode"]], i
        for row, (_, _, blk) in zip(g.decode_block_table, wb["decode"]):
            assert row.tolist() == blk + [-1] * (max_blocks - len(blk)), i
        for row, (_, _, _, blk) in zip(g.prefill_block_table, wb["prefill"]):
            assert row.tolist() == blk + [-1] * (max_blocks - len(blk)), i
        assert g.decode_max_context == max([c for _, c, _ in wb["decode"]], default=0)
        assert g.prefill_total_tokens == sum(t for _, _, t in w.prefill)
        assert g.prefill_max_chunk == max([t for _, _, t in w.prefill], default=0)
        assert g.prefill_max_context == max([s0 + t for _, s0, t in w.prefill], default=0)
        assert g.prefill_cu_chunk_lens[0] == 0
    return len(got)


@pytest.mark.parametrize("name", list(POLICIES))
@pytest.mark.parametrize("seed", range(6))
def test_random_queues_match_oracle(name, seed):
    rng = random.Random(100 + seed)
    n = rng.randrange(1, 60)
    prompts = [rng.randrange(1, 200) for _ in range(n)]
    answers = [rng.randrange(1, 50) for _ in range(n)]
    slots = rng.randrange(1, 17)
    budget = rng.choice([1, 9, 64, 2048])
    max_blocks = 16
    _compare(name, prompts, answers, slots, budget, slots * max_blocks, max_blocks)


@pytest.mark.parametrize("name", ["prefill_first", "decode_first"])
def test_long_prompts_are_chunked_like_the_oracle(name):
    # the head-of-line case: short requests decoding while a long prompt prefills
    prompts, answers = [8, 8, 8, 5000, 30000, 12], [50, 50, 50, 3, 2, 7]
    _compare(name, prompts, answers, 4, 2048, 4 * 2000, 2000)


def test_queue_replay_shape_matches_oracle():
    """1,000 requests at once, prompts 8-32, answers 16-96, 16 slots (the
    aiwithghost page's simulated queue)."""
    rng = np.random.default_rng(7)
    prompts = rng.integers(8, 33, 1000).tolist()
    answers = rng.integers(16, 97, 1000).tolist()
    for name in POLICIES:
        _compare(name, prompts, answers, 16, 2048, 16 * 8, 8)


def test_pool_exhaustion_changes_nothing():
    prompts, answers = [40, 40, 40], [20, 20, 20]
    want = OS.continuous(prompts, answers, 3, 2048, OS.DECODE_FIRST)
    s = kvc.Scheduler(kvc.SCHED_DECODE_FIRST, 3, 2048, 8, 8)   # 3 x 4 blocks needed at most
    for p, a in zip(prompts, answers):
        s.submit(p, a)
    with pytest.raises(kvc.KvcError) as e:
        s.next_step()                 # 3 x 3 blocks for the prompts > 8
    assert e.value.status == -7
    assert s.unfinished() == 3
    with pytest.raises(kvc.KvcError):
        s.next_step()
    # a pool that fits: the plan is the oracle's from the first step on
    s = kvc.Scheduler(kvc.SCHED_DECODE_FIRST, 3, 2048, 12, 8)
    for p, a in zip(prompts, answers):
        s.submit(p, a)
    got = []
    while (st := s.next_step()) is not None:
        got.append(st.decode_ids.tolist())
    assert got == [w.decode for w in want]


def test_submit_rejects_bad_lengths():
    s = kvc.Scheduler(kvc.SCHED_PREFILL_FIRST, 2, 16, 8, 4)
    for p, a in ((0, 1), (1, 0), (64, 2), (60, 6)):     # 64 + 2 - 1 > 4 blocks of 16
        with pytest.raises(kvc.KvcError):
            s.submit(p, a)
    assert s.submit(60, 5) == 0                          # 64 tokens fit exactly
    assert s.next_step() is not None
    for args in ((3, 2, 16, 8, 4), (0, 0, 16, 8, 4), (0, 2, 0, 8, 4), (0, 2, 16, -1, 4),
                 (0, 2, 16, 8, 0)):
        with pytest.raises(kvc.KvcError):
            kvc.Scheduler(*args)


def test_idle_scheduler_builds_nothing():
    s = kvc.Scheduler(kvc.SCHED_STATIC, 4, 16, 8, 4)
    assert s.next_step() is None
    s.submit(5, 1)
    st = s.next_step()
    assert st.first_token_ids.tolist() == [0] and st.finished_ids.tolist() == [0]
    assert s.next_step() is None and s.unfinished() == 0


def test_later_arrivals_join_free_slots():
    """Requests submitted between steps queue behind the earlier ones."""
    s = kvc.Scheduler(kvc.SCHED_DECODE_FIRST, 2, 2048, 16, 4)
    s.submit(4, 3)
    assert s.next_step().prefill_ids.tolist() == [0]
    s.submit(4, 1)
    s.submit(4, 1)
    st = s.next_step()
    assert st.decode_ids.tolist() == [0] and st.prefill_ids.tolist() == [1]
    assert st.finished_ids.tolist() == [1]
    st = s.next_step()
    assert st.decode_ids.tolist() == [0] and st.prefill_ids.tolist() == [2]
    assert sorted(st.finished_ids.tolist()) == [0, 2]
