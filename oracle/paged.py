"""Block-paged cache bookkeeping: slots, the expected pool, gathering back.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The cache lives in fixed-size blocks with a per-sequence block table instead of
one contiguous slab per request (daviddominguez page, section "What prefill
stores and decode reads", on the PagedAttention design; aiwithghost page,
section "How KV cache memory limits concurrency"); blocks are typically 16
tokens (daviddominguez page, section "A prefix already in the cache can skip its
prefill").

Readings (the pages are silent):
* pool layout per layer and per K / V: [num_blocks][num_kv_heads][block_size][head_dim];
* the slot of position p of sequence b is block_table[b][p // bs] * bs + p % bs;
  slot < 0 marks a padding token that writes nothing;
* untouched pool entries keep a sentinel bit pattern (all ones: a NaN in both
  fp32 and bf16), so a stray write or a stray read shows up.

Pins (tests/test_oracle_paged.py): a hand-worked example
(tests/golden/paged_example.json), gather(scatter(x)) == x bitwise, every slot
distinct and in range, and two different block permutations holding the same
sequence gather to the same contiguous cache.
"""
from __future__ import annotations

import numpy as np

SENTINEL16 = np.uint16(0xFFFF)
SENTINEL32 = np.uint32(0xFFFFFFFF)


def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Flat physical slot of logical position ``pos`` of one sequence."""
    return int(block_table_row[pos // block_size]) * block_size + pos % block_size


def slots_for_positions(block_table, seq_ids, positions, block_size: int) -> np.ndarray:
    """Slot of each (sequence, position) pair, int64; one Python step per token."""
    out = np.empty(len(positions), dtype=np.int64)
    for t, (b, p) in enumerate(zip(seq_ids, positions)):
        out[t] = slot_of(block_table[b], int(p), block_size) if p >= 0 else -1
    return out


def empty_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
               bits: int) -> np.ndarray:
    """Pool of raw bit patterns (uint16 for bf16, uint32 for fp32), all sentinel."""
    dt = np.uint16 if bits == 16 else np.uint32
    fill = SENTINEL16 if bits == 16 else SENTINEL32
    return np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=dt)


def scatter(pool: np.ndarray, slots, rows: np.ndarray) -> None:
    """Write token rows [T, Hkv, D] (raw bits, pool dtype) at their slots, in place."""
    bs = pool.shape[2]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        pool[s // bs, :, s % bs, :] = rows[t]


def gather(pool: np.ndarray, block_table_row, n_tokens: int) -> np.ndarray:
    """Positions 0..n_tokens-1 of one sequence, read back through its block table."""
    bs = pool.shape[2]
    out = np.empty((n_tokens, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    for p in range(n_tokens):
        s = slot_of(block_table_row, p, bs)
        out[p] = pool[s // bs, :, s % bs, :]
    return out
