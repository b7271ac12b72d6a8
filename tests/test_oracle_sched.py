"""Pins for oracle.sched: hand-worked traces of each policy, the gouthm page's
head-of-line example, and invariants over random traces. Planted mistakes in
copies of the scheduler each fail a pin."""
import random

import pytest

from oracle import sched as S


def _steps_as_tuples(steps):
    return [(st.decode, st.prefill, st.first_token, st.finished) for st in steps]


def pin_hand_worked(cont=S.continuous, stat=S.static, batches=None):
    p, a = [4, 4, 4], [1, 3, 2]
    # prefill first: decode pauses while a prompt prefills
    got = _steps_as_tuples(cont(p, a, 2, 100, S.PREFILL_FIRST))
    assert got == [([], [(0, 0, 4), (1, 0, 4)], [0, 1], [0]),
                   ([], [(2, 0, 4)], [2], []),
                   ([1, 2], [], [], [2]),
                   ([1], [], [], [1])]
    # decode first: the running row decodes in the step that prefills the new one
    got = _steps_as_tuples(cont(p, a, 2, 100, S.DECODE_FIRST))
    assert got == [([], [(0, 0, 4), (1, 0, 4)], [0, 1], [0]),
                   ([1], [(2, 0, 4)], [2], []),
                   ([1, 2], [], [], [1, 2])]
    # static groups of 2: the finished row idles until the group's longest answer
    got = _steps_as_tuples(stat(p, a, 2))
    assert got == [([], [(0, 0, 4), (1, 0, 4)], [0, 1], [0]),
                   ([1], [], [], []),
                   ([1], [], [], [1]),
                   ([], [(2, 0, 4)], [2], []),
                   ([2], [], [], [2])]


def pin_head_of_line(cont=S.continuous, stat=S.static, batches=None):
    """Three short requests decoding and one 5,000-token prompt, budget 2,048:
    with decode first the short rows decode at every step while the long
    prompt prefills in 2,024 + 2,048 + 928 tokens; with prefill first they
    wait for every chunk (gouthm page, section "The fix that mattered")."""
    p, a = [8, 8, 8, 5000], [50, 50, 50, 2]
    steps = cont(p, a, 4, 2048, S.DECODE_FIRST)
    assert [c for st in steps for c in st.prefill if c[0] == 3] == [(3, 0, 2024), (3, 2024, 2048),
                                                                     (3, 4072, 928)]
    assert all(st.decode[:3] == [0, 1, 2] for st in steps[1:49])
    steps = cont(p, a, 4, 2048, S.PREFILL_FIRST)
    assert [st.decode for st in steps[:4]] == [[], [], [], [0, 1, 2, 3]]
    first, _ = S.first_token_and_finish_steps(steps, 4)
    assert first == [0, 0, 0, 2]


def pin_random_invariants(cont=S.continuous, stat=S.static, batches=None):
    rng = random.Random(3)
    for trial in range(60):
        n = rng.randrange(1, 40)
        p = [rng.randrange(1, 300) for _ in range(n)]
        a = [rng.randrange(1, 40) for _ in range(n)]
        slots, budget = rng.randrange(1, 9), rng.choice([1, 7, 64, 2048])
        for policy in (S.PREFILL_FIRST, S.DECODE_FIRST):
            steps = cont(p, a, slots, budget, policy)
            covered = [0] * n
            gen = [0] * n
            running_max = 0
            for st in steps:
                assert sum(c[2] for c in st.prefill) <= budget
                if policy == S.PREFILL_FIRST:
                    assert not (st.prefill and st.decode)
                rows = {c[0] for c in st.prefill} | set(st.decode)
                running_max = max(running_max, len(rows))
                for r, start, take in st.prefill:
                    assert start == covered[r] and take >= 1
                    covered[r] += take
                for r in st.first_token:
                    assert covered[r] == p[r] and gen[r] == 0
                    gen[r] = 1
                for r in st.decode:
                    assert covered[r] == p[r] and 1 <= gen[r] < a[r]
                    gen[r] += 1
            assert covered == p and gen == a
            assert running_max <= slots
            first, fin = S.first_token_and_finish_steps(steps, n)
            assert all(0 <= f <= g for f, g in zip(first, fin))
            assert first == sorted(first), "admission follows the queue"
        steps = stat(p, a, slots)
        first, fin = S.first_token_and_finish_steps(steps, n)
        assert first == sorted(first) and all(f >= 0 for f in fin)


def pin_blocks_hand_worked(cont=S.continuous, stat=S.static, batches=S.step_batches):
    p, a = [20, 16, 33], [3, 2, 2]
    steps = cont(p, a, 2, 100, S.DECODE_FIRST)
    got = batches(steps, p, a, 10)
    assert got == [
        {"decode": [], "prefill": [(0, 0, 20, [0, 1]), (1, 0, 16, [2])]},
        # request 1's newest token (position 16) opens its second block
        {"decode": [(0, 21, [0, 1]), (1, 17, [2, 3])], "prefill": []},
        # request 1 left after the previous step: its blocks are the lowest free
        {"decode": [(0, 22, [0, 1])], "prefill": [(2, 0, 33, [2, 3, 4])]},
        {"decode": [(2, 34, [2, 3, 4])], "prefill": []}]


def pin_blocks_invariants(cont=S.continuous, stat=S.static, batches=S.step_batches):
    rng = random.Random(5)
    for trial in range(40):
        n = rng.randrange(1, 25)
        p = [rng.randrange(1, 90) for _ in range(n)]
        a = [rng.randrange(1, 30) for _ in range(n)]
        slots, budget = rng.randrange(1, 6), rng.choice([5, 40, 2048])
        steps = cont(p, a, slots, budget, rng.choice([S.PREFILL_FIRST, S.DECODE_FIRST]))
        # brute force: the most blocks live at once, from each step's token counts
        covered, gen, live, peak = [0] * n, [0] * n, {}, 0
        for st in steps:
            for r in st.decode:
                live[r] = -(-(p[r] + gen[r]) // 16)
            for r, s0, t in st.prefill:
                live[r] = -(-(s0 + t) // 16)
            peak = max(peak, sum(live.values()))
            for r, s0, t in st.prefill:
                covered[r] += t
            for r in st.first_token:
                gen[r] = 1
            for r in st.decode:
                gen[r] += 1
            for r in st.finished:
                del live[r]
        got = batches(steps, p, a, peak)
        for b in got:
            rows = [(r, ctx, blk) for r, ctx, blk in b["decode"]] + \
                   [(r, s0 + t, blk) for r, s0, t, blk in b["prefill"]]
            for r, tokens, blk in rows:
                assert len(blk) == -(-tokens // 16) and len(set(blk)) == len(blk)
                assert all(0 <= x < peak for x in blk)
            ids = [x for _, _, blk in rows for x in blk]
            assert len(ids) == len(set(ids)), "a block is held by two requests"
        with pytest.raises(MemoryError):
            batches(steps, p, a, peak - 1)


PINS = [pin_hand_worked, pin_head_of_line, pin_random_invariants, pin_blocks_hand_worked,
        pin_blocks_invariants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---- planted mistakes -------------------------------------------------------

def _lifo(prompts, answers, slots, budget, policy):
    """Admits the newest request first."""
    n = len(prompts)
    order = list(range(n))[::-1]
    steps = S.continuous([prompts[i] for i in order], [answers[i] for i in order], slots, budget,
                         policy)
    m = {i: order[i] for i in range(n)}
    return [S.Step([m[r] for r in st.decode], [(m[r], s, t) for r, s, t in st.prefill],
                   [m[r] for r in st.first_token], [m[r] for r in st.finished]) for st in steps]


def _no_pause(prompts, answers, slots, budget, policy):
    """Never pauses decode, whatever the policy."""
    return S.continuous(prompts, answers, slots, budget, S.DECODE_FIRST)


def _budget_per_row(prompts, answers, slots, budget, policy):
    """Caps each prompt's chunk at the budget instead of the step's total."""
    return S.continuous(prompts, answers, slots, budget * max(1, slots), policy)


def _static_reuses_slots(prompts, answers, group):
    """'Static' that admits into freed slots (that is continuous batching)."""
    return S.continuous(prompts, answers, group, 10 ** 9, S.PREFILL_FIRST)


def _highest_free_first(steps, prompts, answers, num_blocks, block_size=16):
    m = num_blocks - 1
    out = S.step_batches(steps, prompts, answers, num_blocks, block_size)
    for b in out:
        b["decode"] = [(r, c, [m - x for x in blk]) for r, c, blk in b["decode"]]
        b["prefill"] = [(r, s0, t, [m - x for x in blk]) for r, s0, t, blk in b["prefill"]]
    return out


def _context_without_newest(steps, prompts, answers, num_blocks, block_size=16):
    """Sizes a decode row's blocks before its newest token is written."""
    shifted = [S.Step(st.decode, st.prefill, st.first_token, st.finished) for st in steps]
    out = S.step_batches(shifted, [x - 1 if x > 1 else x for x in prompts], answers,
                         num_blocks, block_size)
    return out


def _free_before_prefill(steps, prompts, answers, num_blocks, block_size=16):
    """Returns a leaving decode row's blocks before the same step's prefill
    chunks take theirs."""
    free, held, gen, out = set(range(num_blocks)), {}, {}, []
    for st in steps:
        dec, pf = [], []
        for r in st.decode:
            ctx = prompts[r] + gen[r]
            while len(held.setdefault(r, [])) < -(-ctx // block_size):
                b = min(free)
                free.remove(b)
                held[r].append(b)
            dec.append((r, ctx, list(held[r])))
        for r in st.finished:
            if r in st.decode:
                free.update(held.pop(r))
        for r, s0, t in st.prefill:
            while len(held.setdefault(r, [])) < -(-(s0 + t) // block_size):
                b = min(free)
                free.remove(b)
                held[r].append(b)
            pf.append((r, s0, t, list(held[r])))
        for r in st.first_token:
            gen[r] = 1
        for r in st.decode:
            gen[r] += 1
        for r in st.finished:
            free.update(held.pop(r, []))
        out.append({"decode": dec, "prefill": pf})
    return out


@pytest.mark.parametrize("mutant", [
    dict(cont=_lifo), dict(cont=_no_pause), dict(cont=_budget_per_row),
    dict(stat=_static_reuses_slots), dict(batches=_highest_free_first),
    dict(batches=_context_without_newest), dict(batches=_free_before_prefill)],
    ids=["lifo", "no_pause", "budget_per_row", "static_reuses", "highest_free",
         "ctx_without_newest", "free_before_prefill"])
def test_mutant_fails_a_pin(mutant):
    failed = False
    for pin in PINS:
        try:
            pin(**mutant)
        except (AssertionError, MemoryError, ValueError, KeyError, pytest.fail.Exception):
            failed = True
    assert failed
