"""Planted mistakes in oracle copies (CPU only): each must fail at least one pin.

These show that the pins in tests/oracle_pins.py would catch a plausible slip in
the oracle: a wrong scale, a wrong head map, a dropped self-attention term,
swapped K/V, a wrong normaliser, an off-by-one in the causal window, a
transposed slot formula.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import paged
from tests import oracle_pins as P


def _attend(q, k, v, scale, *, head_map=lambda h, G, Hkv: h // G, window=lambda n: n,
            swap=False, norm="sum", scale_fn=None, q_head=lambda h, g: h):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if swap:
        k, v = v, k
    hq, d = q.shape
    n, hkv, _ = k.shape
    G = hq // hkv
    sc = scale if scale_fn is None else scale_fn(d)
    out = np.empty((hq, d))
    m_ = window(n)
    for h in range(hq):
        g = head_map(h, G, hkv)
        s = sc * (k[:m_, g, :] @ q[q_head(h, g)])
        p = np.exp(s - s.max())
        out[h] = (p @ v[:m_, g, :]) / (p.sum() if norm == "sum" else p.max())
    return out


MUTANTS = {
    "scale_1_over_D": lambda q, k, v, s: _attend(q, k, v, s, scale_fn=lambda d: 1.0 / d),
    "head_map_modulo": lambda q, k, v, s: _attend(q, k, v, s, head_map=lambda h, G, Hkv: h % Hkv),
    "drops_self": lambda q, k, v, s: _attend(q, k, v, s, window=lambda n: max(n - 1, 0)),
    "swapped_k_v": lambda q, k, v, s: _attend(q, k, v, s, swap=True),
    "max_normaliser": lambda q, k, v, s: _attend(q, k, v, s, norm="max"),
    "query_of_group": lambda q, k, v, s: _attend(q, k, v, s, q_head=lambda h, g: g),
}


def _all_attend_pins(f):
    """True when every attend_row pin passes."""
    try:
        checks = [
            P.err_vs_sdpa(f) < 1e-12,
            P.single_key_exact(f),
            P.uniform_is_mean(f) < 1e-14,
            P.two_key_logistic(f) < 1e-13,
            P.needle_retrieval(f) < 1e-9,
            P.gqa_equals_repeated_mha(f) == 0.0,
        ]
    except Exception:
        return False
    return all(checks)


def test_unmutated_copy_passes():
    assert _all_attend_pins(lambda q, k, v, s: _attend(q, k, v, s))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with np.errstate(all="ignore"):
        assert not _all_attend_pins(MUTANTS[name])


def test_prefill_off_by_one_is_caught():
    def shifted(q_chunk, k_seq, v_seq, prefix, scale):
        return np.stack([A.attend_row(q_chunk[i], k_seq[:max(prefix + i, 1)],
                                      v_seq[:max(prefix + i, 1)], scale)
                         for i in range(q_chunk.shape[0])])
    assert P.prefill_err_vs_sdpa(shifted) > 1e-3


def test_transposed_slot_formula_is_caught():
    def bad_slot(row, pos, bs):
        return int(row[pos % bs]) * bs + pos // bs if pos % bs < len(row) else -1
    assert not P.golden_slots_ok(bad_slot)


def test_slot_off_by_one_block_is_caught():
    class Bad:
        empty_pool = staticmethod(paged.empty_pool)
        scatter = staticmethod(paged.scatter)

        @staticmethod
        def slots_for_positions(bt, seq_ids, positions, bs):
            return np.array([int(bt[b][p // bs]) * bs + (p + 1) % bs
                             for b, p in zip(seq_ids, positions)], np.int64)

        gather = staticmethod(paged.gather)
    assert not P.gather_scatter_roundtrip(Bad)


def _positions(q_rows, k_seq, v_seq, positions, scale, *, reach=0, head_map=None):
    """attend_positions with a planted slip: the window ends `reach` keys off, or
    the query head reads another kv head."""
    q = np.asarray(q_rows, np.float64)
    pos = np.asarray(positions)
    n = int(pos.max()) + 1
    k, v = np.asarray(k_seq[:n], np.float64), np.asarray(v_seq[:n], np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    out = np.empty(q.shape)
    for h in range(hq):
        g = (h // (hq // hkv)) if head_map is None else head_map(h, hkv)
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s[np.arange(n)[None, :] > pos[:, None] + reach] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("kw", [dict(reach=-1), dict(reach=1), dict(head_map=lambda h, hkv: h % hkv)])
def test_position_rows_mutant_is_caught(kw):
    with np.errstate(all="ignore"):
        assert not P.positions_err_vs_sdpa(lambda *a: _positions(*a, **kw)) < 1e-12


def test_position_rows_unmutated_copy_passes():
    assert P.positions_err_vs_sdpa(_positions) < 1e-12
