"""Queue replay host logic (kv_cache_decode_append_amd.replay): interpolation,
summed shares, and the replay's timings against closed forms and the oracle
scheduler's plans. No GPU."""
import numpy as np
import pytest

import workloads as W
from oracle import sched as OS

kvc = pytest.importorskip("kv_cache_decode_append_amd")
from kv_cache_decode_append_amd import replay as R  # noqa: E402


def test_interp2_exact_on_grid_and_bilinear_between():
    xs, ys = [1, 2, 4], [8, 16, 32, 64]
    t = np.array([[x * 100 + y for y in ys] for x in xs], np.float64)
    for i, x in enumerate(xs):
        for j, y in enumerate(ys):
            assert R.interp2(xs, ys, t, x, y) == t[i, j]
    # the table is linear in both axes, so bilinear interpolation is exact
    assert R.interp2(xs, ys, t, 3, 40) == pytest.approx(340)
    # a product table: bilinear at the cell centre is the mean of the corners
    p = np.outer([1.0, 3.0], [2.0, 10.0])
    assert R.interp2([0, 1], [0, 1], p, 0.5, 0.5) == pytest.approx(np.mean(p))
    for x, y in ((0, 8), (5, 8), (1, 7), (1, 65)):
        with pytest.raises(ValueError):
            R.interp2(xs, ys, t, x, y)


def _linear_times(a_dec=0.01, b_dec=1e-4, a_pf=0.02, b_pf=3e-4):
    rows, lengths = [1, 2, 4, 8, 16], [1, 8, 32, 64, 128]
    dec = [[a_dec * n + b_dec * n * c for c in lengths] for n in rows]
    pf = [[a_pf * n + b_pf * n * L for L in lengths] for n in rows]
    return R.StepTimes(rows, lengths, dec, pf)


def test_summed_shares_of_a_linear_table():
    """With step time linear in length, the summed-shares estimate of mixed
    lengths equals the time of the same rows at their mean length."""
    times = _linear_times()
    s = kvc.Scheduler(kvc.SCHED_PREFILL_FIRST, 4, 2048, 64, 16)
    for p, a in ((10, 3), (30, 3), (50, 3), (90, 3)):
        s.submit(p, a)
    prefill = s.next_step()
    assert R.step_cost_ms(prefill, times) == pytest.approx(times.prefill(4, 45))
    dec = s.next_step()
    assert list(dec.decode_context_lens) == [11, 31, 51, 91]
    assert R.step_cost_ms(dec, times) == pytest.approx(times.decode(4, 46))
    assert R.step_cost_ms(dec, times, recompute=True) == pytest.approx(times.prefill(4, 46))


def _unit_times():
    rows, lengths = [1, 16], [1, 4096]
    return R.StepTimes(rows, lengths, [[1.0, 1.0], [1.0, 1.0]], [[1.0, 1.0], [1.0, 1.0]])


def test_one_at_a_time_closed_form():
    """Unit step costs: request i's first token is ready after
    sum_{j<i} a_j + 1 steps, the queue is done after sum a_j steps."""
    prompts, answers = W.queue_requests(50, seed=3)
    for pol in R.queue_policies()[:2]:
        steps = R.plan(pol, prompts, answers)
        res = R.replay(steps, [R.step_cost_ms(s, _unit_times(), pol.recompute) for s in steps],
                       len(prompts))
        before = np.concatenate([[0], np.cumsum(answers)[:-1]])
        assert np.array_equal(res["ttft_ms"], before + 1.0)
        assert res["all_done_ms"] == sum(answers)


@pytest.mark.parametrize("which", [2, 3, 4])
def test_batched_policies_count_the_oracle_steps(which):
    """Unit step costs: TTFT of each request is the oracle's step index + 1."""
    prompts, answers = W.queue_requests(200, seed=4)
    pol = R.queue_policies()[which]
    if pol.sched == kvc.SCHED_STATIC:
        want = OS.static(prompts, answers, pol.slots)
    else:
        oracle_policy = OS.DECODE_FIRST if pol.sched == kvc.SCHED_DECODE_FIRST else OS.PREFILL_FIRST
        want = OS.continuous(prompts, answers, pol.slots, 2048, oracle_policy)
    first, fin = OS.first_token_and_finish_steps(want, len(prompts))
    steps = R.plan(pol, prompts, answers)
    res = R.replay(steps, [1.0] * len(steps), len(prompts))
    assert np.array_equal(res["ttft_ms"], np.array(first) + 1.0)
    assert np.array_equal(res["done_ms"], np.array(fin) + 1.0)


def test_static_group_time_is_its_longest_answer():
    prompts, answers = [8] * 6, [3, 9, 2, 5, 5, 1]
    pol = R.Policy("static 3", kvc.SCHED_STATIC, 3)
    steps = R.plan(pol, prompts, answers)
    res = R.replay(steps, [1.0] * len(steps), 6)
    assert res["all_done_ms"] == 9 + 5
    assert res["ttft_ms"].tolist() == [1, 1, 1, 10, 10, 10]


def test_summary_columns():
    res = {"ttft_ms": np.arange(1, 101, dtype=np.float64) * 1e3, "all_done_ms": 200e3}
    s = R.summarize(res, 1000)
    assert s["median_ttft_s"] == 50.5 and s["p95_ttft_s"] == pytest.approx(95.05)
    assert s["all_done_s"] == 200 and s["tokens_per_s"] == 5


def test_queue_workload_ranges():
    p, a = W.queue_requests()
    assert len(p) == len(a) == 1000
    assert min(p) == 8 and max(p) == 32 and min(a) == 16 and max(a) == 96
