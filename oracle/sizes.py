"""KV-cache size and capacity arithmetic.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: aiwithghost page, section "How KV cache memory limits concurrency"
(bytes per token = 2 x layers x KV heads x head size x bytes per number);
daviddominguez page, section "What prefill stores and decode reads" (the same
formula, the 128 KiB per token figure, and the capacity division: free memory /
bytes per token = tokens, tokens / tokens per request = requests).

Pins: tests/test_oracle_sizes.py against the numbers the pages print
(tests/golden/page_numbers.json).
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Raw K+V storage for one token of one request across all layers."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def tokens_that_fit(free_bytes: int, bytes_per_token: int) -> int:
    return free_bytes // bytes_per_token


def requests_that_fit(tokens: int, tokens_per_request: int) -> int:
    return tokens // tokens_per_request


def pool_bytes(num_blocks: int, kv_heads: int, block_size: int, head_dim: int,
               dtype_bytes: int) -> int:
    """Bytes of one layer's K pool plus V pool of ``num_blocks`` blocks."""
    return 2 * num_blocks * kv_heads * block_size * head_dim * dtype_bytes


def projection_rows_uncached(prompt: int, answer: int) -> int:
    """Token rows projected by the loop that reruns the whole sequence.

    Pass n (1..answer) runs over prompt + n - 1 tokens. Counted by summing the
    passes, not by the page's closed form, so the two can be compared.
    """
    return sum(prompt + n - 1 for n in range(1, answer + 1))


def projection_rows_cached(prompt: int, answer: int) -> int:
    """Token rows projected with a cache: the prompt once, then one row for each
    generated token that is fed back (the last one is not)."""
    return prompt + sum(1 for _ in range(1, answer))
