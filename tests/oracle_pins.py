"""Pin checks for the oracle, written against references other than the oracle.

Each check takes the function under test as an argument so that
tests/test_oracle_mutations.py can run the same checks on oracle copies with a
planted mistake and confirm that at least one check fails for each mistake.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- references
def sdpa_causal_rows(q, k, v, prefix: int, scale: float) -> np.ndarray:
    """torch CPU scaled_dot_product_attention (fp64, GQA) for query rows at
    positions prefix .. prefix+C-1 over keys 0 .. prefix+C-1.

    q: [C, Hq, D]; k, v: [prefix+C, Hkv, D].
    """
    c = q.shape[0]
    n = k.shape[0]
    assert n == prefix + c
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]   # [1,Hq,C,D]
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2)[None]
    mask = torch.arange(n)[None, :] <= (prefix + torch.arange(c))[:, None]  # bottom-right causal
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                         enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


def sdpa_default_scale_rows(q, k, v) -> np.ndarray:
    """Same, full causal attention from position 0, with torch's default scale."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2)[None]
    out = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- attend_row pins
def err_vs_sdpa(attend_row, seed=0) -> float:
    """Max |f - sdpa| over full causal rows, several (G, D, n) shapes."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for hkv, g, d, n in [(1, 1, 16, 9), (2, 2, 16, 17), (2, 4, 64, 33), (4, 1, 8, 5),
                         (1, 8, 32, 20), (3, 2, 128, 12)]:
        hq = hkv * g
        q, k, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
        scale = 1.0 / math.sqrt(d)
        ref = sdpa_default_scale_rows(q, k, v)
        got = np.stack([attend_row(q[i], k[:i + 1], v[:i + 1], scale) for i in range(n)])
        worst = max(worst, float(np.nanmax(np.abs(got - ref))) if np.all(np.isfinite(got)) else math.inf)
    return worst


def single_key_exact(attend_row) -> bool:
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 8, 32), _rand(rng, 1, 2, 32), _rand(rng, 1, 2, 32)
    try:
        o = attend_row(q, k, v, 0.3)
    except Exception:
        return False
    return bool(np.array_equal(o, np.repeat(v[0], 4, axis=0)))


def uniform_is_mean(attend_row) -> float:
    rng = np.random.default_rng(2)
    n, d = 37, 16
    q = np.zeros((6, d))
    k, v = _rand(rng, n, 3, d), _rand(rng, n, 3, d)
    o = attend_row(q, k, v, 0.25)
    ref = np.repeat(v.mean(axis=0), 2, axis=0)
    return float(np.max(np.abs(o - ref)))


def two_key_logistic(attend_row) -> float:
    """Two keys: the weight on key 1 is the logistic function of the logit gap."""
    rng = np.random.default_rng(3)
    worst = 0.0
    for _ in range(20):
        d = 8
        q, k, v = _rand(rng, 1, d), _rand(rng, 2, 1, d), _rand(rng, 2, 1, d)
        scale = rng.uniform(0.1, 1.0)
        gap = scale * float(np.dot(q[0], k[1, 0]) - np.dot(q[0], k[0, 0]))
        w1 = 1.0 / (1.0 + math.exp(-gap))
        ref = (1.0 - w1) * v[0, 0] + w1 * v[1, 0]
        worst = max(worst, float(np.max(np.abs(attend_row(q, k, v, scale)[0] - ref))))
    return worst


def needle_retrieval(attend_row) -> float:
    """A key aligned with the query and a logit 30+ above the rest returns its value."""
    rng = np.random.default_rng(4)
    n, hkv, g, d = 300, 2, 4, 64
    scale = 1.0 / math.sqrt(d)
    k, v = _rand(rng, n, hkv, d) * 0.1, _rand(rng, n, hkv, d)
    q = np.repeat(_rand(rng, hkv, d)[:, None, :], g, axis=1).reshape(hkv * g, d)
    j = 123
    for kh in range(hkv):
        qh = q[kh * g]
        alpha = 40.0 / (scale * float(qh @ qh))
        k[j, kh] = alpha * qh
    o = attend_row(q, k, v, scale)
    ref = np.repeat(v[j], g, axis=0)
    return float(np.max(np.abs(o - ref)))


def gqa_equals_repeated_mha(attend_row) -> float:
    rng = np.random.default_rng(5)
    n, hkv, g, d = 21, 2, 4, 16
    q, k, v = _rand(rng, hkv * g, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    a = attend_row(q, k, v, 0.25)
    b = attend_row(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.25)
    return float(np.max(np.abs(a - b)))


# ---------------------------------------------------------------- prefill pins
def prefill_err_vs_sdpa(prefill_chunk_rows, seed=6) -> float:
    rng = np.random.default_rng(seed)
    worst = 0.0
    for hkv, g, d, prefix, c in [(2, 4, 32, 0, 7), (1, 2, 16, 17, 16), (2, 1, 64, 33, 5),
                                 (1, 4, 16, 40, 1)]:
        hq = hkv * g
        q = _rand(rng, c, hq, d)
        k, v = _rand(rng, prefix + c, hkv, d), _rand(rng, prefix + c, hkv, d)
        scale = 1.0 / math.sqrt(d)
        ref = sdpa_causal_rows(q, k, v, prefix, scale)
        got = prefill_chunk_rows(q, k, v, prefix, scale)
        worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


def positions_err_vs_sdpa(attend_positions, seed=9) -> float:
    """Rows at given positions (a whole chunk, and a scattered subset of one)
    against torch SDPA with the bottom-right causal mask."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for hkv, g, d, prefix, c in [(2, 4, 32, 0, 7), (1, 2, 16, 17, 16), (2, 1, 64, 33, 5),
                                 (1, 4, 16, 40, 1), (2, 4, 16, 90, 40)]:
        hq = hkv * g
        q = _rand(rng, c, hq, d)
        k, v = _rand(rng, prefix + c, hkv, d), _rand(rng, prefix + c, hkv, d)
        scale = 1.0 / math.sqrt(d)
        ref = sdpa_causal_rows(q, k, v, prefix, scale)
        got = attend_positions(q, k, v, prefix + np.arange(c), scale)
        worst = max(worst, float(np.max(np.abs(got - ref))))
        sub = np.sort(rng.choice(c, size=max(1, c // 3), replace=False))
        got = attend_positions(q[sub], k, v, prefix + sub, scale)
        worst = max(worst, float(np.max(np.abs(got - ref[sub]))))
    return worst


# ---------------------------------------------------------------- paged pins
def golden_slots_ok(slot_of) -> bool:
    with open(os.path.join(GOLD, "paged_example.json")) as f:
        e = json.load(f)
    got = [slot_of(e["block_table_row"], p, e["block_size"]) for p in e["positions"]]
    return got == e["slots"]


def gather_scatter_roundtrip(paged, seed=8) -> bool:
    """Scatter a sequence through a permuted block table, gather it back."""
    rng = np.random.default_rng(seed)
    nb, hkv, bs, d = 12, 3, 16, 8
    n = 70                                              # 5 blocks, last one partial
    rows = rng.integers(0, 2 ** 16 - 1, size=(n, hkv, d), dtype=np.uint16)
    bt = rng.permutation(nb)[:5]
    pool = paged.empty_pool(nb, hkv, bs, d, 16)
    slots = paged.slots_for_positions([bt], [0] * n, np.arange(n), bs)
    if len(set(slots.tolist())) != n or slots.min() < 0 or slots.max() >= nb * bs:
        return False
    paged.scatter(pool, slots, rows)
    if not np.array_equal(paged.gather(pool, bt, n), rows):
        return False
    # untouched blocks and the unused tail of the last block keep the sentinel
    touched = np.zeros(nb * bs, bool)
    touched[slots] = True
    flat = pool.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    return bool(np.all(flat[~touched] == 0xFFFF))
