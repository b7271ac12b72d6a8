"""Seeded synthetic inputs for the paged KV-cache decode/append path.

This module is shared by the CPU oracle and by the GPU tests/bench. It only
draws random numbers and lays out integer bookkeeping inputs (context lengths,
block tables). It holds none of the attention arithmetic, no slot computation
and no cache layout logic: those live separately in `oracle/` and in the HIP
library.

Workloads (shapes taken from the pages' workloads):

* ``C1`` toy single sequence, fp32: 4 q-heads / 4 kv-heads, head_dim 16,
  block 16; a 16-token prompt and a 48-token answer (aiwithghost.com, "KV cache
  and continuous batching: 1,000 people ask AI", section "Why does writing one
  token at a time repeat work?", P = 16, N = 48).
* ``C2`` continuous batch of 16 sequences, fp32, 8/8 heads, head_dim 64,
  context 64 (same page, section "What our lab measured", decode step at
  context 64 with 16 rows).
* ``C3`` Llama-3.1-8B attention shape, bf16: 32 q / 8 kv heads, head_dim 128,
  batch 64, context uniform in [2000, 2300] (daviddominguez.dev, "The KV cache
  and prefix caching", section "What prefill stores and decode reads": 2,000
  prompt tokens, 2,300 at the end of generation, 64 requests).
* ``C4`` skewed mix: 210 sequences (the same page's capacity estimate),
  lognormal context lengths with median 6,000 and a tail clipped at 32,000
  (gouthm.com, "The KV cache is not your bottleneck", section "The setup"),
  some rows mid-prefill with 2,048-token chunks (section "The fix that
  mattered").
* ``C5`` long context: 8 sequences at 32,000 tokens decode, plus a 2,048-token
  prefill chunk per sequence over a 30,000-token cached prefix.
* ``P1`` prefix caching, C3's attention shape: a 2,000-token prompt whose first
  1,800 tokens (system instructions and examples) are shared with a cached
  prompt (daviddominguez.dev, section "A prefix already in the cache can skip
  its prefill"); ``shared_prompts`` builds such token lists and
  ``prefix_values`` gives each position values that depend on its whole token
  prefix, as a model's keys and values do.

Seeds: workload k draws sequence b's values from ``default_rng([k, b])`` in the
order K, V (all positions), then Q; the block permutation from
``default_rng([k, 999999])``; context lengths from ``default_rng([k, 888888])``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16
BLOCK_SEED = 999999
LENGTH_SEED = 888888


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace
    B: int                   # sequences
    Hq: int
    Hkv: int
    D: int
    dtype: str               # "fp32" | "bf16"
    sigma: float             # values ~ N(0, 1) * sigma
    layers: int = 1          # layers the step is reported over
    block_size: int = BLOCK_SIZE


C1 = Workload("C1-toy-fp32", 1, B=1, Hq=4, Hkv=4, D=16, dtype="fp32", sigma=1.0)
C1_PROMPT = 16
C1_ANSWER = 48
C1_POOL_BLOCKS = 8

C2 = Workload("C2-batch16-fp32", 2, B=16, Hq=8, Hkv=8, D=64, dtype="fp32", sigma=1.0)
C2_CTX = 64
C2_POOL_BLOCKS = 128

C3 = Workload("C3-llama8b-gqa-b64-ctx2k", 3, B=64, Hq=32, Hkv=8, D=128, dtype="bf16",
              sigma=0.5, layers=32)
C3_CTX_LO, C3_CTX_HI = 2000, 2300
C3_POOL_BLOCKS = 64 * 2300 // BLOCK_SIZE     # 9,200 blocks: 64 x 2,300 tokens

C4 = Workload("C4-skewed-b210", 4, B=210, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
C4_MEDIAN = 6000
C4_SIGMA_LN = math.log(5.0) / 2.3263478740408408   # p99 = 5 x median = 30,000
C4_CLIP = 32000
C4_PREFILL_ROWS = 4
C4_CHUNK = 2048

C5 = Workload("C5-long-b8-ctx32k", 5, B=8, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
C5_CTX = 32000
C5_PREFIX = 30000
C5_CHUNK = 2048

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(n_tokens) // block_size)


def context_lengths(w: Workload) -> np.ndarray:
    """Per-sequence token counts held in the cache after this step's writes."""
    rng = np.random.default_rng([w.wid, LENGTH_SEED])
    if w.wid == 1:
        return np.array([C1_PROMPT + C1_ANSWER - 1], dtype=np.int64)
    if w.wid == 2:
        return np.full(w.B, C2_CTX, dtype=np.int64)
    if w.wid == 3:
        return rng.integers(C3_CTX_LO, C3_CTX_HI + 1, size=w.B).astype(np.int64)
    if w.wid == 4:
        x = rng.lognormal(mean=math.log(C4_MEDIAN), sigma=C4_SIGMA_LN, size=w.B)
        return np.clip(np.rint(x), 1, C4_CLIP).astype(np.int64)
    if w.wid == 5:
        return np.full(w.B, C5_CTX, dtype=np.int64)
    raise ValueError(w)


def c4_prefill_rows(ctx: np.ndarray) -> np.ndarray:
    """Rows of the skewed mix that are mid-prefill this step (seeded choice
    among rows long enough to hold a 2,048-token chunk over a >= 2,048 prefix)."""
    rng = np.random.default_rng([C4.wid, LENGTH_SEED, 1])
    eligible = np.flatnonzero(ctx >= 2 * C4_CHUNK)
    return np.sort(rng.choice(eligible, size=C4_PREFILL_ROWS, replace=False))


def block_tables(w: Workload, ctx: np.ndarray, num_blocks: int,
                 max_blocks: int | None = None, seed_extra: int = 0) -> np.ndarray:
    """Physical blocks handed out in random order from a seeded pool.

    Sequence b takes the next ceil(ctx_b / block_size) ids of a seeded
    permutation of ``range(num_blocks)``. Unused table entries hold -1.
    """
    need = [blocks_for(c, w.block_size) for c in ctx]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {sum(need)}")
    if max_blocks is None:
        max_blocks = max(need) if need else 0
    rng = np.random.default_rng([w.wid, BLOCK_SEED, seed_extra])
    perm = rng.permutation(num_blocks)
    bt = np.full((len(ctx), max_blocks), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[cur:cur + n]
        cur += n
    return bt


def sequence_values(w: Workload, b: int, n_kv: int, n_q: int,
                    q_positions_draw: int | None = None):
    """fp32 K, V of ``n_kv`` positions and Q of ``n_q`` positions for sequence b.

    K, V: [n_kv, Hkv, D]; Q: [n_q, Hq, D]; values N(0, 1) * sigma, fp32 (not
    yet rounded to the cache dtype).
    """
    rng = np.random.default_rng([w.wid, b])
    k = (rng.standard_normal((n_kv, w.Hkv, w.D), dtype=np.float32) * np.float32(w.sigma))
    v = (rng.standard_normal((n_kv, w.Hkv, w.D), dtype=np.float32) * np.float32(w.sigma))
    q = (rng.standard_normal((n_q, w.Hq, w.D), dtype=np.float32) * np.float32(w.sigma))
    return k, v, q


def small_workload(name: str, wid: int, B: int, Hq: int, Hkv: int, D: int, dtype: str,
                   sigma: float = 1.0) -> Workload:
    """Ad-hoc workload for parity grids (seed namespace ``wid`` >= 100)."""
    return Workload(name, wid, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, sigma=sigma)


P1 = Workload("P1-prefix-bf16", 6, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5, layers=32)
P1_PROMPT = 2000
P1_SHARED = 1800
PREFIX_VOCAB = 128000


def shared_prompts(n_prompts: int, shared: int = P1_SHARED, length: int = P1_PROMPT,
                   seed: int = 0) -> list[list[int]]:
    """Token id lists that agree on their first ``shared`` tokens."""
    rng = np.random.default_rng([P1.wid, 777777, seed])
    stem = rng.integers(0, PREFIX_VOCAB, shared).tolist()
    return [stem + rng.integers(0, PREFIX_VOCAB, length - shared).tolist()
            for _ in range(n_prompts)]


def _prefix_seeds(tokens) -> list[int]:
    """One 63-bit seed per position, a running mix of the tokens up to it."""
    h, out = 0x2545F4914F6CDD1D, []
    for t in tokens:
        h = ((h ^ (int(t) + 0x9E3779B97F4A7C15)) * 0x100000001B3) & ((1 << 64) - 1)
        out.append(h >> 1)
    return out


def prefix_values(w: Workload, tokens) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """k, v [n, Hkv, D] and q [n, Hq, D] (float32, N(0, 1) * sigma): position p's
    values are drawn from a generator seeded by tokens[0..p], so two prompts
    with the same opening have the same values there."""
    n = len(tokens)
    k = np.empty((n, w.Hkv, w.D), np.float32)
    v = np.empty_like(k)
    q = np.empty((n, w.Hq, w.D), np.float32)
    for p, sd in enumerate(_prefix_seeds(tokens)):
        rng = np.random.default_rng([w.wid, sd])
        k[p] = rng.standard_normal((w.Hkv, w.D), dtype=np.float32) * w.sigma
        v[p] = rng.standard_normal((w.Hkv, w.D), dtype=np.float32) * w.sigma
        q[p] = rng.standard_normal((w.Hq, w.D), dtype=np.float32) * w.sigma
    return k, v, q


# ---- request queue (aiwithghost page, section "What our lab measured") -------

QUEUE_SEED = 777777
QUEUE_N = 1000
QUEUE_SLOTS = 16
QUEUE_PROMPT = (8, 32)     # inclusive ranges
QUEUE_ANSWER = (16, 96)


def queue_requests(n: int = QUEUE_N, seed: int = QUEUE_SEED):
    """Prompt and answer lengths of ``n`` requests, all arriving at t = 0, drawn
    uniformly from the inclusive ranges the lab's simulated queue states."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(QUEUE_PROMPT[0], QUEUE_PROMPT[1] + 1, n)
    answers = rng.integers(QUEUE_ANSWER[0], QUEUE_ANSWER[1] + 1, n)
    return prompts.astype(np.int64).tolist(), answers.astype(np.int64).tolist()
