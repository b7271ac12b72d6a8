"""Attention over a KV cache: the definition, the naive loop and the cached loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Arithmetic is fp64 on the values the caller passes (for a bf16 cache those are
the bf16-rounded values, exactly upcast). The pages fix no arithmetic precision;
they only keep the cache in 16-bit numbers.

What is computed (aiwithghost page, section "Why does writing one token at a
time repeat work?": each token is projected into a query, a key and a value; the
new token's query is compared with the keys of all earlier tokens and the
result weights their values; the Transformer paper's scaled dot product):

    row(t, h):  s_j = scale * <q_t[h], k_j[g(h)]>      j = 0 .. t
                p_j = exp(s_j - max_j s_j)
                o   = sum_j p_j v_j[g(h)] / sum_j p_j

with scale = 1/sqrt(D) unless given, and grouped-query sharing g(h) = h // G,
G = Hq / Hkv, so that consecutive query heads share one K/V head
(daviddominguez page, section "What prefill stores and decode reads", on
grouped-query attention). Causality (same page, opening section): position t
sees positions 0..t, itself included, never a later one.

Readings where the pages are silent:
* the softmax scale is 1/sqrt(D) (scaled dot product), passed explicitly;
* q-head h uses K/V head h // G (contiguous groups);
* a decode step appends first, then attends over everything stored, so the
  new token attends to itself (daviddominguez page, section "What prefill
  stores and decode reads": append, then attend the new query over everything
  stored).

Pins (tests/test_oracle_attention.py): torch CPU scaled_dot_product_attention in
fp64 with GQA; closed forms (one key gives its value exactly; equal logits give
the mean of V; two keys give the logistic weighting); needle retrieval; the
pages' "identical tokens on both paths" (cached == uncached, bitwise); the pages'
row counts 1,896 vs 63; immutability of earlier rows.
"""
from __future__ import annotations

import math

import numpy as np


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def attend_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One query position over a prefix of keys/values.

    q: [Hq, D]; k, v: [n, Hkv, D] (positions 0..n-1 the query may see).
    Returns o: [Hq, D] in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    n, hkv, d2 = k.shape
    assert d == d2 and v.shape == k.shape and n >= 1 and hq % hkv == 0
    group = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = scale * (k[:, g, :] @ q[h])          # [n] logits
        m = s.max()
        p = np.exp(s - m)                         # unnormalised weights
        out[h] = (p @ v[:, g, :]) / p.sum()
    return out


def causal_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, first: int, last: int,
                scale: float) -> np.ndarray:
    """Rows first..last (inclusive) of full causal attention over one sequence.

    q: [>= last+1, Hq, D] (position-indexed); k, v: [>= last+1, Hkv, D].
    Row i sees positions 0..i. Returns [last-first+1, Hq, D].
    """
    return np.stack([attend_row(q[i], k[:i + 1], v[:i + 1], scale)
                     for i in range(first, last + 1)])


def generate_uncached(q, k, v, prompt: int, answer: int, scale: float):
    """The loop that reruns the whole sequence at every step.

    daviddominguez page, section "What prefill stores and decode reads" (the
    hand-written loop that passes the whole sequence to the model again on each
    iteration); aiwithghost page, section "Why does writing one token at a time
    repeat work?". Pass n = 1..answer runs over positions 0..prompt+n-2,
    recomputing every position's K/V row and the full causal attention of every
    row, and keeps the last row: that row yields answer token n.

    Returns (outputs [answer, Hq, D], kv_rows_computed, attention_rows_computed).
    """
    outs = []
    kv_rows = 0
    att_rows = 0
    for n in range(1, answer + 1):
        last = prompt + n - 2
        k_pass = np.array(k[:last + 1], copy=True)       # recomputed each pass
        v_pass = np.array(v[:last + 1], copy=True)
        kv_rows += last + 1
        rows = causal_rows(q, k_pass, v_pass, 0, last, scale)
        att_rows += last + 1
        outs.append(rows[-1])
    return np.stack(outs), kv_rows, att_rows


def generate_cached(q, k, v, prompt: int, answer: int, scale: float):
    """The loop with a contiguous per-sequence KV cache.

    Prefill writes the prompt's K/V once; each later pass appends one position's
    K/V to the cache and attends that position's query over everything stored
    (aiwithghost page, section "What does a KV cache keep?"; daviddominguez
    page, section "What prefill stores and decode reads").

    Returns (outputs [answer, Hq, D], kv_rows_computed, cache [prompt+answer-1, Hkv, D] x2).
    """
    hkv, d = k.shape[1], k.shape[2]
    cache_k = np.empty((0, hkv, d), dtype=np.asarray(k).dtype)
    cache_v = np.empty((0, hkv, d), dtype=np.asarray(v).dtype)
    outs = []
    kv_rows = 0
    # prefill: the prompt's K/V once, then the prompt's last row
    cache_k = np.concatenate([cache_k, k[:prompt]])
    cache_v = np.concatenate([cache_v, v[:prompt]])
    kv_rows += prompt
    outs.append(attend_row(q[prompt - 1], cache_k, cache_v, scale))
    for n in range(2, answer + 1):
        t = prompt + n - 2                                  # the new position
        cache_k = np.concatenate([cache_k, k[t:t + 1]])     # append ...
        cache_v = np.concatenate([cache_v, v[t:t + 1]])
        kv_rows += 1
        outs.append(attend_row(q[t], cache_k, cache_v, scale))   # ... then attend
    return np.stack(outs), kv_rows, (cache_k, cache_v)


def attend_positions(q_rows, k_seq, v_seq, positions, scale: float) -> np.ndarray:
    """Query rows of one sequence at absolute positions `positions`, each over
    keys 0 .. its position (the causal window of attend_row), computed for all
    rows of a query head at once: logits scale * Q K^T, keys past a row's
    position removed, row-wise softmax, then weights times V. The same
    definition as attend_row in matrix form, for checking many rows over long
    prefixes (a whole query tile or chunk).

    q_rows: [R, Hq, D]; k_seq, v_seq: [>= max(positions) + 1, Hkv, D];
    positions: [R] ints. Returns [R, Hq, D] in fp64.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    n = int(pos.max()) + 1
    k = np.asarray(k_seq[:n], dtype=np.float64)
    v = np.asarray(v_seq[:n], dtype=np.float64)
    r, hq, d = q.shape
    hkv = k.shape[1]
    assert pos.shape == (r,) and pos.min() >= 0 and hq % hkv == 0 and k.shape[2] == d
    group = hq // hkv
    outside = np.arange(n)[None, :] > pos[:, None]            # [R, n] keys a row may not see
    out = np.empty((r, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)                 # [R, n] logits
        s[outside] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))           # unnormalised weights
        out[:, h, :] = (p @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def decode_rows(q_new, k_seqs, v_seqs, scale: float) -> np.ndarray:
    """One decode step for a batch of sequences of mixed lengths.

    q_new: [B, Hq, D] (each sequence's newest position); k_seqs[b], v_seqs[b]:
    [ctx_b, Hkv, D], already holding the newest position (append first).
    Returns [B, Hq, D].
    """
    return np.stack([attend_row(q_new[b], k_seqs[b], v_seqs[b], scale)
                     for b in range(len(k_seqs))])


def prefill_chunk_rows(q_chunk, k_seq, v_seq, prefix: int, scale: float) -> np.ndarray:
    """Rows prefix .. prefix+C-1 of one sequence, over its cached prefix plus
    the chunk's own earlier positions (a prefill step capped at a token budget,
    gouthm.com page, section "The fix that mattered"; prefill that starts after
    a cached prefix, daviddominguez page, section "A prefix already in the cache
    can skip its prefill").

    q_chunk: [C, Hq, D]; k_seq, v_seq: [>= prefix+C, Hkv, D]. Returns [C, Hq, D].
    """
    return np.stack([attend_row(q_chunk[i], k_seq[:prefix + i + 1], v_seq[:prefix + i + 1], scale)
                     for i in range(q_chunk.shape[0])])
