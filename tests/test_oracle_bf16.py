"""Pins for oracle/bf16.py: hand-worked tie cases and torch's CPU conversion."""
import os

import numpy as np
import torch

from oracle import bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden", "bf16_cases.txt")


def _cases():
    rows = []
    with open(GOLD) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()[:2]
            rows.append((int(a, 16), int(b, 16)))
    return rows


def test_hand_worked_cases():
    cases = _cases()
    assert len(cases) >= 10
    f32 = np.array([a for a, _ in cases], dtype=np.uint32).view(np.float32)
    got = bf16.to_bf16_bits(f32)
    want = np.array([b for _, b in cases], dtype=np.uint16)
    assert np.array_equal(got, want), [(hex(a), hex(int(g)), hex(b))
                                       for (a, b), g in zip(cases, got) if g != b]


def test_matches_torch_cpu_conversion():
    rng = np.random.default_rng(7)
    # wide exponent range plus dense ties around 1.0
    x = rng.standard_normal(200_000).astype(np.float32) * np.exp2(
        rng.integers(-40, 40, 200_000)).astype(np.float32)
    ties = (np.arange(0x3F800000, 0x3F800000 + 65536 * 4, 0x4000, dtype=np.uint32)
            | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.to_bf16_bits(x), want)


def test_roundtrip_exact_for_bf16_values():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)          # positive finite bf16 patterns
    assert np.array_equal(bf16.to_bf16_bits(bf16.bits_to_f32(bits)), bits)
