"""fp32 -> bfloat16 rounding, written from the format's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 keeps the top 16 bits of an IEEE-754 binary32 value (sign, 8 exponent
bits, 7 fraction bits). Rounding to nearest, ties to even, adds half a unit of
the last kept place minus one, plus the kept LSB, to the 32-bit pattern and then
truncates. The pages keep the cache in "16-bit numbers" / bfloat16 (aiwithghost
page, section "How KV cache memory limits concurrency"; daviddominguez page,
section "What prefill stores and decode reads"). Only finite inputs are
generated.

Pin: tests/test_oracle_bf16.py compares against torch's CPU conversion and
against hand-worked tie cases in tests/golden/bf16_cases.txt.
"""
from __future__ import annotations

import numpy as np


def to_bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of RNE(bf16(x)) for finite fp32 ``x``."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bits_to_f32(bits) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x) -> np.ndarray:
    """fp32 array whose values are ``x`` rounded to bfloat16 (RNE)."""
    return bits_to_f32(to_bf16_bits(x))
