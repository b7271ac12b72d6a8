"""Iteration-level scheduling of a request queue: which rows decode and which
prompt chunks prefill at each step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is scheduled (aiwithghost page "KV cache and continuous batching: 1,000
people ask AI", sections "How does continuous batching share the server?" and
"What our lab measured"; gouthm page "The KV cache is not your bottleneck",
section "The fix that mattered"):

* continuous batching rebuilds the batch at every step: a request that has its
  last token leaves at once and the next request in the queue is admitted, in
  queue order, into the free slot and starts with its prefill;
* the prefill of a prompt yields the answer's first token; every later token
  takes one decode step of that row;
* static batching starts a group of requests together and decodes until the
  longest answer in the group is done; finished rows sit idle in their slots
  and the next group starts only after that;
* the lab's simulator pauses decode while any admitted prompt is prefilling
  (``PREFILL_FIRST``); the gouthm page's fix gives decode strict priority and
  lets prefill fill a fixed token budget per step, chunking long prompts
  (``DECODE_FIRST``: every row that can decode does so at every step, and the
  step's prefill chunks, taken in admission order, add up to at most the
  budget).

Readings (the pages are silent):

* admission happens at the start of a step, before the step's batch is built;
* a step's prefill token budget counts prompt tokens only (decode rows are one
  token each and always run under ``DECODE_FIRST``); under ``PREFILL_FIRST``
  the same budget caps the prefill-only steps;
* a request whose answer has one token leaves right after its prefill;
* static groups prefill all their prompts in their first step, budget aside.

Pins (tests/test_oracle_sched.py): hand-worked traces for each policy, the
gouthm page's head-of-line example (decode never waits under DECODE_FIRST, it
waits for every chunk of a long prompt under PREFILL_FIRST), queue-order
admission, and token conservation on random traces.
"""
from __future__ import annotations

import dataclasses

PREFILL_FIRST = 0
DECODE_FIRST = 1


@dataclasses.dataclass
class Step:
    decode: list          # request ids decoding one token, in admission order
    prefill: list         # (request id, first prompt position, tokens), in admission order
    first_token: list     # ids whose first token comes out of this step
    finished: list        # ids that leave after this step


def continuous(prompts, answers, slots: int, budget: int, policy: int) -> list:
    """Steps of continuous batching for requests 0..n-1 queued in that order."""
    n = len(prompts)
    assert len(answers) == n and slots >= 1 and budget >= 1
    assert all(p >= 1 for p in prompts) and all(a >= 1 for a in answers)
    queue = list(range(n))
    running = []                       # admission order
    done_prefill = [0] * n
    generated = [0] * n
    steps = []
    while queue or running:
        while queue and len(running) < slots:
            running.append(queue.pop(0))
        pending = [r for r in running if done_prefill[r] < prompts[r]]
        ready = [r for r in running if done_prefill[r] == prompts[r] and generated[r] < answers[r]]
        decode = []
        chunks = []
        if policy == DECODE_FIRST or not pending:
            decode = ready
        if policy == DECODE_FIRST or pending:
            left = budget
            for r in pending:
                if left == 0:
                    break
                take = min(prompts[r] - done_prefill[r], left)
                chunks.append((r, done_prefill[r], take))
                left -= take
        first, finished = [], []
        for r, start, take in chunks:
            done_prefill[r] += take
            if done_prefill[r] == prompts[r]:
                generated[r] = 1
                first.append(r)
        for r in decode:
            generated[r] += 1
        for r in list(running):
            if done_prefill[r] == prompts[r] and generated[r] == answers[r]:
                finished.append(r)
                running.remove(r)
        steps.append(Step(decode, chunks, first, finished))
    return steps


def static(prompts, answers, group: int) -> list:
    """Steps of static batching: groups of ``group`` requests in queue order."""
    n = len(prompts)
    steps = []
    for g0 in range(0, n, group):
        members = list(range(g0, min(n, g0 + group)))
        generated = {r: 1 for r in members}
        steps.append(Step([], [(r, 0, prompts[r]) for r in members], list(members),
                          [r for r in members if answers[r] == 1]))
        for _ in range(max(answers[r] for r in members) - 1):
            decode = [r for r in members if generated[r] < answers[r]]
            for r in decode:
                generated[r] += 1
            steps.append(Step(decode, [], [], [r for r in decode if generated[r] == answers[r]]))
    return steps


def first_token_and_finish_steps(steps, n: int):
    """Index of the step that yields each request's first token, and of the
    step after which it leaves."""
    first = [-1] * n
    fin = [-1] * n
    for i, st in enumerate(steps):
        for r in st.first_token:
            first[r] = i
        for r in st.finished:
            fin[r] = i
    return first, fin


def _blocks_for(tokens: int, block_size: int) -> int:
    return (tokens + block_size - 1) // block_size


def step_batches(steps, prompts, answers, num_blocks: int, block_size: int = 16) -> list:
    """The kernel inputs of each step: which cache blocks each row reads and
    writes.

    A request holds the blocks its tokens occupy: before a step runs, each row
    of the step (decode rows first, then prefill chunks, each in the order the
    step lists them) takes the lowest-numbered free blocks until it holds
    ceil(tokens / block_size) of them, counting the tokens the step writes;
    after the step, every request that leaves returns all of its blocks (the
    paged layout of the aiwithghost page's memory section; block order and
    timing are readings). A decode row of a request with a prompt of p tokens
    and g tokens generated so far writes the K/V of its newest token at
    position p + g - 1 and attends over p + g positions.

    Returns, per step, ``{"decode": [(id, context_len, blocks)], "prefill":
    [(id, start, take, blocks)]}`` with ``blocks`` the request's block list
    after the step's allocation. Raises ``MemoryError`` when the pool runs out.
    """
    n = len(prompts)
    free = set(range(num_blocks))
    held = [[] for _ in range(n)]
    covered = [0] * n
    gen = [0] * n
    out = []

    def grow(r, tokens):
        need = _blocks_for(tokens, block_size) - len(held[r])
        if need > len(free):
            raise MemoryError("KV block pool exhausted")
        for _ in range(max(0, need)):
            b = min(free)
            free.remove(b)
            held[r].append(b)

    for st in steps:
        dec, pf = [], []
        for r in st.decode:
            ctx = prompts[r] + gen[r]
            grow(r, ctx)
            dec.append((r, ctx, list(held[r])))
        for r, start, take in st.prefill:
            assert start == covered[r]
            grow(r, start + take)
            pf.append((r, start, take, list(held[r])))
        for r, start, take in st.prefill:
            covered[r] += take
        for r in st.first_token:
            gen[r] = 1
        for r in st.decode:
            gen[r] += 1
        for r in st.finished:
            free.update(held[r])
            held[r] = []
        out.append({"decode": dec, "prefill": pf})
    return out
