"""Queue replay from measured step times.

The aiwithghost page's lab ("KV cache and continuous batching: 1,000 people ask
AI", section "What our lab measured") times the model directly and then
replays a queue of 1,000 requests that all arrive at t = 0 using only those
step times, interpolated inside the measured grid; a batch of rows with mixed
lengths is estimated by summing shares of equal-length measurements (each of
n rows costs 1/n of an n-row step at its own length). This module does the
same with the native scheduler's plans (include/kvc_sched.h) and a table of
step times measured on the GPU:

* ``StepTimes``: milliseconds of one decode step (n rows, every row at context
  c) and of one prefill step (n prompts of L tokens each, nothing cached) over
  a grid of (n, c) and (n, L), with bilinear interpolation inside the grid;
* ``plan``: the scheduler's steps for a policy;
* ``replay``: the time at which each request's first token is ready (TTFT,
  measured from the common arrival at t = 0) and at which the last request is
  done, from the steps' estimated costs.

Policies (the page's table, plus the gouthm page's decode-first lanes):
one at a time without a cache (every token recomputes the whole prompt and
answer so far as a prefill of that length), one at a time with the cache,
static batches, continuous batching with decode paused during prefill (the
lab's simulator), and continuous batching with decode first and a prefill
token budget ("The KV cache is not your bottleneck", section "The fix that
mattered").

Host code: it plans and sums; the step times come from kernels timed on the
GPU by the caller.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from ._lib import SCHED_DECODE_FIRST, SCHED_PREFILL_FIRST, SCHED_STATIC, Scheduler

BLOCK = 16


def interp2(xs, ys, table, x: float, y: float) -> float:
    """Bilinear interpolation of table[i][j] (measured at xs[i], ys[j]) at
    (x, y); raises outside the grid."""
    xs, ys = np.asarray(xs, np.float64), np.asarray(ys, np.float64)
    if not (xs[0] <= x <= xs[-1] and ys[0] <= y <= ys[-1]):
        raise ValueError(f"({x}, {y}) lies outside the measured grid")
    i = min(int(np.searchsorted(xs, x, side="right")) - 1, len(xs) - 2) if len(xs) > 1 else 0
    j = min(int(np.searchsorted(ys, y, side="right")) - 1, len(ys) - 2) if len(ys) > 1 else 0
    tx = 0.0 if len(xs) == 1 else (x - xs[i]) / (xs[i + 1] - xs[i])
    ty = 0.0 if len(ys) == 1 else (y - ys[j]) / (ys[j + 1] - ys[j])
    t = np.asarray(table, np.float64)
    i1, j1 = min(i + 1, len(xs) - 1), min(j + 1, len(ys) - 1)
    return float((1 - tx) * (1 - ty) * t[i, j] + tx * (1 - ty) * t[i1, j] +
                 (1 - tx) * ty * t[i, j1] + tx * ty * t[i1, j1])


@dataclasses.dataclass
class StepTimes:
    rows: list              # batch rows measured, ascending
    lengths: list           # contexts (decode) and prompt lengths (prefill), ascending
    decode_ms: list         # [len(rows)][len(lengths)]
    prefill_ms: list        # [len(rows)][len(lengths)]

    def decode(self, n: int, ctx: int) -> float:
        return interp2(self.rows, self.lengths, self.decode_ms, n, ctx)

    def prefill(self, n: int, length: int) -> float:
        return interp2(self.rows, self.lengths, self.prefill_ms, n, length)


@dataclasses.dataclass
class Policy:
    name: str
    sched: int              # SCHED_* policy of the native scheduler
    slots: int
    recompute: bool = False  # no cache: a decode row re-runs its whole prefix as a prefill


def queue_policies(slots: int = 16) -> list:
    return [Policy("one at a time, no cache", SCHED_PREFILL_FIRST, 1, recompute=True),
            Policy("one at a time, KV cache", SCHED_PREFILL_FIRST, 1),
            Policy(f"static batches of {slots}, cache", SCHED_STATIC, slots),
            Policy(f"continuous batching, {slots} slots", SCHED_PREFILL_FIRST, slots),
            Policy(f"continuous batching, {slots} slots, decode first", SCHED_DECODE_FIRST,
                   slots)]


def plan(policy: Policy, prompts, answers, budget: int = 2048) -> list:
    """The native scheduler's steps for every request queued at once."""
    max_blocks = max((p + a - 1 + BLOCK - 1) // BLOCK for p, a in zip(prompts, answers))
    s = Scheduler(policy.sched, policy.slots, budget, policy.slots * max_blocks, max_blocks)
    for p, a in zip(prompts, answers):
        s.submit(int(p), int(a))
    steps = []
    while (st := s.next_step()) is not None:
        steps.append(st)
    return steps


def step_cost_ms(st, times: StepTimes, recompute: bool = False) -> float:
    """Estimated milliseconds of one step: summed shares of equal-length
    measurements, decode rows and prefill chunks as separate launches."""
    cost = 0.0
    n = len(st.decode_ids)
    if n:
        if recompute:
            cost += sum(times.prefill(n, int(c)) for c in st.decode_context_lens) / n
        else:
            cost += sum(times.decode(n, int(c)) for c in st.decode_context_lens) / n
    m = len(st.prefill_ids)
    if m:
        if np.any(st.prefill_prefix_lens != 0):
            raise ValueError("chunks over a cached prefix are outside the measured grid")
        takes = np.diff(st.prefill_cu_chunk_lens)
        cost += sum(times.prefill(m, int(t)) for t in takes) / m
    return cost


def replay(steps, costs_ms, n_requests: int) -> dict:
    """TTFT of every request (end of the step that makes its first token) and
    the time the last request is done, from per-step costs; all requests
    arrive at t = 0."""
    ttft = np.full(n_requests, np.nan)
    done = np.full(n_requests, np.nan)
    t = 0.0
    for st, c in zip(steps, costs_ms):
        t += c
        ttft[st.first_token_ids] = t
        done[st.finished_ids] = t
    if np.isnan(ttft).any() or np.isnan(done).any():
        raise ValueError("a request never got its first token or never finished")
    return {"ttft_ms": ttft, "done_ms": done, "all_done_ms": float(done.max())}


def summarize(result: dict, answer_tokens: int) -> dict:
    """The page's table columns: median and p95 TTFT, all-done time (seconds),
    answer tokens per second over the whole queue. p95 is numpy's default
    (linear) percentile."""
    ttft = result["ttft_ms"] / 1e3
    all_done = result["all_done_ms"] / 1e3
    return {"median_ttft_s": float(np.median(ttft)), "p95_ttft_s": float(np.percentile(ttft, 95)),
            "all_done_s": all_done, "tokens_per_s": answer_tokens / all_done}
