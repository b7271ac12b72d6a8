"""Pins for oracle/attention.py and oracle/paged.py (CPU only)."""
import json
import math
import os

import numpy as np

import workloads as W
from oracle import attention as A
from oracle import bf16, paged
from tests import oracle_pins as P

with open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")) as f:
    PAGE = json.load(f)


def test_matches_torch_sdpa_fp64():
    assert P.err_vs_sdpa(A.attend_row) < 1e-12


def test_single_key_returns_its_value_exactly():
    assert P.single_key_exact(A.attend_row)


def test_equal_logits_give_mean_of_values():
    assert P.uniform_is_mean(A.attend_row) < 1e-14


def test_two_keys_logistic_closed_form():
    assert P.two_key_logistic(A.attend_row) < 1e-13


def test_needle_retrieval():
    # exp(-30) * 300 keys ~ 3e-11 of leakage
    assert P.needle_retrieval(A.attend_row) < 1e-9


def test_gqa_equals_mha_with_repeated_heads():
    assert P.gqa_equals_repeated_mha(A.attend_row) == 0.0


def test_prefill_rows_match_sdpa_with_offset_mask():
    assert P.prefill_err_vs_sdpa(A.prefill_chunk_rows) < 1e-12


def test_position_rows_match_sdpa_with_offset_mask():
    assert P.positions_err_vs_sdpa(A.attend_positions) < 1e-12


def test_paged_golden_slots():
    assert P.golden_slots_ok(paged.slot_of)


def test_paged_gather_scatter_roundtrip():
    assert P.gather_scatter_roundtrip(paged)


def _c1_values():
    k, v, q = W.sequence_values(W.C1, 0, W.C1_PROMPT + W.C1_ANSWER, W.C1_PROMPT + W.C1_ANSWER)
    return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)


def test_cached_equals_uncached_bitwise_and_row_counts():
    """Identical results on both paths, and the pages' 1,896 vs 63 rows."""
    q, k, v = _c1_values()
    e = PAGE["projection_rows"]
    scale = A.default_scale(W.C1.D)
    out_u, rows_u, att_rows = A.generate_uncached(q, k, v, e["prompt"], e["answer"], scale)
    out_c, rows_c, (ck, cv) = A.generate_cached(q, k, v, e["prompt"], e["answer"], scale)
    assert rows_u == e["uncached"] and rows_c == e["cached"]
    assert att_rows == e["uncached"]
    assert np.array_equal(out_u, out_c)
    assert ck.shape[0] == e["prompt"] + e["answer"] - 1 == 63
    assert np.array_equal(ck, k[:63]) and np.array_equal(cv, v[:63])


def test_earlier_rows_never_change():
    """Causality: row i is bitwise the same whenever it is computed."""
    q, k, v = _c1_values()
    scale = A.default_scale(W.C1.D)
    at_40 = A.causal_rows(q, k[:41], v[:41], 0, 40, scale)
    at_63 = A.causal_rows(q, k, v, 0, 63, scale)
    assert np.array_equal(at_40, at_63[:41])


def test_chunked_prefill_equals_one_shot_and_decode():
    rng = np.random.default_rng(11)
    n, hkv, g, d = 80, 2, 4, 32
    q, k, v = (rng.standard_normal((n, hkv * g, d)), rng.standard_normal((n, hkv, d)),
               rng.standard_normal((n, hkv, d)))
    s = A.default_scale(d)
    one = A.prefill_chunk_rows(q, k, v, 0, s)
    parts = [A.prefill_chunk_rows(q[a:b], k, v, a, s) for a, b in [(0, 16), (16, 45), (45, 80)]]
    assert np.array_equal(one, np.concatenate(parts))
    # a 1-token chunk is a decode step
    dec = A.decode_rows(q[None, 50], [k[:51]], [v[:51]], s)
    assert np.array_equal(A.prefill_chunk_rows(q[50:51], k, v, 50, s), dec)


def test_decode_rows_mixed_lengths_match_sdpa():
    rng = np.random.default_rng(12)
    hkv, g, d = 2, 4, 16
    lens = [1, 5, 16, 17, 33]
    ks = [rng.standard_normal((n, hkv, d)) for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    qs = rng.standard_normal((len(lens), hkv * g, d))
    s = A.default_scale(d)
    got = A.decode_rows(qs, ks, vs, s)
    for b, n in enumerate(lens):
        ref = P.sdpa_causal_rows(qs[b:b + 1], ks[b], vs[b], n - 1, s)[0]
        assert np.max(np.abs(got[b] - ref)) < 1e-12


def test_bf16_inputs_are_exact_in_fp64():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = bf16.round_bf16(x)
    assert np.array_equal(r.astype(np.float64).astype(np.float32), r)
    assert np.max(np.abs(r - x) / np.abs(x)) <= 2.0 ** -8


def test_workload_block_tables_are_a_permutation():
    ctx = W.context_lengths(W.C3)
    assert ctx.min() >= W.C3_CTX_LO and ctx.max() <= W.C3_CTX_HI
    bt = W.block_tables(W.C3, ctx, W.C3_POOL_BLOCKS)
    used = np.concatenate([bt[b, :W.blocks_for(c)] for b, c in enumerate(ctx)])
    assert len(np.unique(used)) == len(used)
    assert used.min() >= 0 and used.max() < W.C3_POOL_BLOCKS


def test_c4_lengths_shape_the_pages_mix():
    ctx = W.context_lengths(W.C4)
    assert len(ctx) == 210 and ctx.min() >= 1 and ctx.max() <= W.C4_CLIP
    assert 4500 < np.median(ctx) < 8000          # median around 6k
    assert ctx.max() > 20000                      # a long tail
    rows = W.c4_prefill_rows(ctx)
    assert len(rows) == W.C4_PREFILL_ROWS and np.all(ctx[rows] >= 2 * W.C4_CHUNK)
    assert math.isclose(np.exp(W.C4_SIGMA_LN * 2.3263478740408408), 5.0)
