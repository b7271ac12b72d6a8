"""The launch-route rule of StepRunner (kv_cache_decode_append_amd/step.py),
on the CPU with an injected timer: single-kind steps take the separate
calls; a mixed step's size class is timed on both routes, alternating, for a
warm-up step and `trials` counted steps each, then keeps the one launch only
if it beat the separate launches by more than the margin; a decided class
never changes route.
"""
import pytest

from kv_cache_decode_append_amd.step import ONE_LAUNCH, SEPARATE, StepRunner


def test_size_classes_are_powers_of_two_at_or_above():
    assert StepRunner.size_class(206, 31_999, 8_192) == (256, 32_768, 8_192)
    assert StepRunner.size_class(1, 1, 1) == (1, 1, 1)
    assert StepRunner.size_class(0, 0, 0) == (0, 0, 0)
    assert StepRunner.size_class(129, 2_049, 2_047) == (256, 4_096, 2_048)


def test_single_kind_steps_take_the_separate_calls():
    r = StepRunner(32)
    assert r.pick(64, 2_300, 0) == (SEPARATE, None)
    assert r.pick(0, 0, 2_048) == (SEPARATE, None)
    assert r.samples == {} and r.decisions == {}


def _drive(r, times, n=20, sizes=(206, 32_000, 8_192)):
    """Runs the rule over n steps of one size class with route times `times`."""
    routes = []
    for _ in range(n):
        route, key = r.pick(*sizes)
        routes.append(route)
        if key is not None:
            r.record(key, route, times[route])
    return routes


@pytest.mark.parametrize("one_ms,expect", [(2.30, ONE_LAUNCH), (2.44, SEPARATE), (2.60, SEPARATE),
                                           (2.44 * 0.985, SEPARATE)])
def test_mixed_class_is_timed_then_decided(one_ms, expect):
    r = StepRunner(32, trials=3, margin=0.02)
    routes = _drive(r, {SEPARATE: 2.44, ONE_LAUNCH: one_ms})
    # calibration alternates, starting with the separate launches: a warm-up
    # and 3 counted steps on each route
    assert routes[:8] == [SEPARATE, ONE_LAUNCH] * 4
    assert set(routes[8:]) == {expect}
    assert r.decisions == {StepRunner.size_class(206, 32_000, 8_192): expect}


def test_decision_uses_medians_and_never_changes():
    r = StepRunner(32, trials=3, margin=0.0)
    route, key = r.pick(16, 100, 64)
    assert (route, key) == (SEPARATE, StepRunner.size_class(16, 100, 64))
    # the warm-ups (50 ms, 0.1 ms) are not counted; one slow outlier on the
    # separate route does not move its median
    for ms in (50.0, 1.0, 9.0, 1.1):
        r.record(key, SEPARATE, ms)
    for ms in (0.1, 1.2, 1.2):
        r.record(key, ONE_LAUNCH, ms)
    assert key not in r.decisions             # two counted one-launch samples so far
    r.record(key, ONE_LAUNCH, 1.2)
    assert r.decisions[key] == SEPARATE       # median 1.1 against 1.2
    for _ in range(5):
        assert r.pick(16, 100, 64) == (SEPARATE, None)


def test_classes_are_independent():
    r = StepRunner(32, trials=1)
    a, b = (8, 100, 64), (64, 2_000, 2_048)
    _drive(r, {SEPARATE: 1.0, ONE_LAUNCH: 0.5}, n=6, sizes=a)
    _drive(r, {SEPARATE: 1.0, ONE_LAUNCH: 1.5}, n=6, sizes=b)
    assert r.decisions == {StepRunner.size_class(*a): ONE_LAUNCH,
                           StepRunner.size_class(*b): SEPARATE}


def test_fixed_routes_and_argument_checks():
    assert StepRunner(32, route=ONE_LAUNCH).pick(1, 1, 1) == (ONE_LAUNCH, None)
    assert StepRunner(32, route=SEPARATE).pick(64, 2_000, 2_048) == (SEPARATE, None)
    with pytest.raises(ValueError):
        StepRunner(32, route="fastest")
    with pytest.raises(ValueError):
        StepRunner(32, trials=0)
