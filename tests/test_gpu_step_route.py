"""GPU: StepRunner (kv_cache_decode_append_amd/step.py), the caller-side rule
that runs a continuous-batching step by separate launches or by one launch.

The same step (decode rows plus prefill chunks; its writes are idempotent, so
it can run again on the same pool) goes through a runner in "auto" mode:
its first steps alternate the two routes while they are timed (a warm-up
and `trials` counted steps each), then the class keeps one. Every run's rows
are checked against the oracle and the pool against the inputs bit for bit;
runs on one route give the same bits; the prefill rows are the same bits on
both routes; a single-kind step takes the separate calls without being
timed.
"""
import numpy as np
import pytest
import torch

from tests.gpu_cases import assert_close, say
from tests.test_gpu_mixed import MixedCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _parts(inp):
    dec = dict(q=inp["q_decode"], k_new=inp["k_new"], v_new=inp["v_new"],
               block_table=inp["decode_block_table"], context_lens=inp["decode_context_lens"],
               max_context=inp["decode_max_context"])
    pf = dict(q=inp["q_prefill"], k=inp["k_prefill"], v=inp["v_prefill"],
              cu_chunk_lens=inp["cu_chunk_lens"], prefix_lens=inp["prefix_lens"],
              block_table=inp["prefill_block_table"], max_chunk=inp["prefill_max_chunk"])
    return dec, pf


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_auto_route_times_both_then_keeps_one(kvc, dtype):
    D = 128 if dtype == "bf16" else 32
    case = MixedCase(f"route-{dtype}", 9500 + D, 32 if dtype == "bf16" else 8, 8 if dtype == "bf16"
                     else 2, D, dtype, dec_ctx=[1, 17, 300, 2_000, 5_000, 64],
                     pf_prefix=[0, 700], pf_chunk=[300, 129])
    say(f"step route {dtype}: 6 decode rows + 2 chunks, auto, 2 trials per route, 9 runs")
    cache = case.fill(kvc)
    dec, pf = _parts(case.inputs())
    runner = kvc.StepRunner(case.w.Hq, trials=2)
    routes, outs = [], []
    for _ in range(9):
        route, _ = runner.pick(dec["q"].shape[0], dec["max_context"], pf["q"].shape[0])
        out_dec, out_pf = runner.run(cache, dec, pf)
        torch.cuda.synchronize()
        routes.append(route)
        outs.append((out_dec.clone(), out_pf.clone()))
        case.check(cache, out_dec, out_pf)
    assert routes[:6] == [kvc.SEPARATE, kvc.ONE_LAUNCH] * 3
    key = runner.size_class(dec["q"].shape[0], dec["max_context"], pf["q"].shape[0])
    assert set(routes[6:]) == {runner.decisions[key]}
    say(f"  decided {runner.decisions[key]}: separate {runner.samples[key][kvc.SEPARATE]} ms, "
        f"one launch {runner.samples[key][kvc.ONE_LAUNCH]} ms")
    ib = torch.int16 if dtype == "bf16" else torch.int32
    by_route = {}
    for r, (od, op) in zip(routes, outs):
        if r in by_route:                          # same route, same bits
            assert torch.equal(od.view(ib), by_route[r][0].view(ib))
            assert torch.equal(op.view(ib), by_route[r][1].view(ib))
        by_route.setdefault(r, (od, op))
    sep, one = by_route[kvc.SEPARATE], by_route[kvc.ONE_LAUNCH]
    assert torch.equal(sep[1].view(ib), one[1].view(ib)), "prefill rows differ between routes"
    assert_close(one[0].float().cpu().numpy(), sep[0].float().cpu().numpy().astype(np.float64),
                 dtype, "decode rows: one launch vs separate")


def test_single_kind_steps_are_not_timed(kvc):
    case = MixedCase("route-single", 9600, 32, 8, 128, "bf16", dec_ctx=[40, 3_000],
                     pf_prefix=[100], pf_chunk=[64])
    say("step route: decode-only and prefill-only steps take the separate calls")
    cache = case.fill(kvc)
    dec, pf = _parts(case.inputs())
    runner = kvc.StepRunner(case.w.Hq, trials=1, timer=lambda fn: pytest.fail("timed"))
    out_dec, none = runner.run(cache, dec, None)
    none2, out_pf = runner.run(cache, None, pf)
    torch.cuda.synchronize()
    assert none is None and none2 is None and runner.samples == {}
    case.check(cache, out_dec, out_pf)
