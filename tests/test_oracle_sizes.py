"""Pins for oracle/sizes.py against the numbers the pages print."""
import json
import os

from oracle import sizes

with open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")) as f:
    PAGE = json.load(f)


def test_bytes_per_token():
    e = PAGE["kv_bytes_per_token"]
    assert sizes.kv_bytes_per_token(**e["args"]) == e["value"]
    assert sizes.kv_bytes_per_token(**e["args"]) == PAGE["kib_per_token"]["value"] * 1024


def test_32_kv_heads():
    e = PAGE["kv_heads_32_kib_per_token"]
    assert sizes.kv_bytes_per_token(**e["args"]) == e["value"] * 1024


def test_request_sizes():
    per = sizes.kv_bytes_per_token(32, 8, 128, 2)
    e = PAGE["request_4096_tokens_mib"]
    assert per * e["tokens"] == e["value"] * 2 ** 20
    e = PAGE["prompt_2000_mib"]
    assert per * e["tokens"] / 2 ** 20 == e["value_from_formula"]
    assert per * e["tokens"] / 2 ** 20 != e["value_printed"]      # the page's misprint
    e = PAGE["end_2300_mib"]
    assert per * e["tokens"] / 2 ** 20 == e["value"]
    e = PAGE["requests_64_gib"]
    assert round(per * e["tokens"] * e["requests"] / 2 ** 30, e["decimals"]) == e["value_printed"]


def test_capacity_arithmetic():
    e = PAGE["capacity"]
    per = sizes.kv_bytes_per_token(32, 8, 128, 2)
    toks = sizes.tokens_that_fit(e["free_gib"] * 2 ** 30, per)
    assert abs(toks - e["tokens_approx"]) / e["tokens_approx"] < 0.01
    reqs = sizes.requests_that_fit(toks, e["tokens_per_request"])
    assert abs(reqs - e["requests_approx"]) <= 5


def test_projection_rows():
    e = PAGE["projection_rows"]
    assert sizes.projection_rows_uncached(e["prompt"], e["answer"]) == e["uncached"]
    assert sizes.projection_rows_cached(e["prompt"], e["answer"]) == e["cached"]
    # the page's closed forms N*P + N(N-1)/2 and P + N - 1, over a grid
    for p in range(1, 20):
        for n in range(1, 30):
            assert sizes.projection_rows_uncached(p, n) == n * p + n * (n - 1) // 2
            assert sizes.projection_rows_cached(p, n) == p + n - 1


def test_pool_bytes_c3():
    # 64 sequences x 2,300 tokens in 16-token blocks, one layer, bf16, 8 kv heads, D 128
    nb = 64 * 2300 // 16
    assert sizes.pool_bytes(nb, 8, 16, 128, 2) == 64 * 2300 * sizes.kv_bytes_per_token(1, 8, 128, 2)
    assert sizes.pool_bytes(nb, 8, 16, 128, 2) == 301_465_600 * 2
