"""GPU: calls with nothing to do return at once, with empty outputs and the
cache bitwise unchanged; a zero-length chunk inside a prefill batch writes and
attends nothing for its sequence while the others are computed as usual."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_cases import PrefillCase, assert_close, device_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float8_e4m3fn])
def test_zero_sized_calls(kvc, dtype):
    say(f"zero-sized calls through every entry point, {dtype}")
    dev = "cuda"
    Hkv, Hq, D = 2, 4, 64
    act = torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype
    cache = kvc.PagedKVCache.allocate(8, Hkv, D, dtype, fill_bits=-1)
    k0, v0 = cache.k_cache.clone(), cache.v_cache.clone()
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32, device=dev)
    x = lambda *s: torch.zeros(*s, dtype=act, device=dev)
    bt2 = i32(2, 4)
    # no tokens to place or write
    slots = kvc.slot_mapping(bt2, 8, i32(0), i32(0), err_flag=cache.err_flag)
    assert slots.shape == (0,) and slots.dtype == torch.int64
    kvc.kv_append(cache, slots, x(0, Hkv, D), x(0, Hkv, D))
    # no sequences to decode
    out = kvc.paged_decode_attention(cache, x(0, Hq, D), i32(0, 4), i32(0), 0)
    assert out.shape == (0, Hq, D)
    out = kvc.decode_append_attention(cache, x(0, Hq, D), x(0, Hkv, D), x(0, Hkv, D), i32(0, 4),
                                      i32(0), 0)
    assert out.shape == (0, Hq, D)
    # no sequences to prefill, and two sequences whose chunks are both empty
    out = kvc.chunked_prefill_attention(cache, x(0, Hq, D), x(0, Hkv, D), x(0, Hkv, D), i32(1),
                                        i32(0), i32(0, 4), 0)
    assert out.shape == (0, Hq, D)
    prefix = torch.tensor([3, 0], dtype=torch.int32, device=dev)
    for mcl in (None, 3):
        out = kvc.chunked_prefill_attention(cache, x(0, Hq, D), x(0, Hkv, D), x(0, Hkv, D), i32(3),
                                            prefix, bt2, 0, max_context_len=mcl)
        assert out.shape == (0, Hq, D)
    # a mixed step with neither part (the one-launch kernel takes fp32 caches at head_dim 32 only)
    if dtype != torch.float32:
        assert kvc.mixed_step_attention(cache, Hq) == (None, None)
    torch.cuda.synchronize()
    assert torch.equal(cache.k_cache.view(torch.uint8), k0.view(torch.uint8))
    assert torch.equal(cache.v_cache.view(torch.uint8), v0.view(torch.uint8))
    assert int(cache.err_flag.item()) == 0


@pytest.mark.parametrize("dtype,d,g", [("bf16", 128, 4), ("bf16", 64, 2), ("fp32", 64, 1)])
@pytest.mark.parametrize("split", [False, True])
def test_empty_chunks_inside_a_batch(kvc, dtype, d, g, split):
    say(f"prefill batch with zero-length chunks, {dtype} D={d} G={g} split={split}")
    w = W.small_workload(f"pf-empty-{dtype}-{d}-{g}", 995 + d + g, B=5, Hq=2 * g, Hkv=2, D=d,
                         dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0)
    prefix = [30, 50, 0, 17, 0]
    chunk = [20, 0, 33, 0, 1]
    case = PrefillCase(w, prefix, chunk, 60)
    mcl = max(p + c for p, c in zip(prefix, chunk)) if split else None
    cache, out = case.run_gpu(kvc, max_context_len=mcl)
    assert int(cache.err_flag.item()) == 0
    pk, pv = case.oracle_pool()
    assert np.array_equal(device_bits(cache.k_cache), pk), "K pool differs"
    assert np.array_equal(device_bits(cache.v_cache), pv), "V pool differs"
    got = out.float().cpu().numpy()
    assert got.shape[0] == sum(chunk)
    for i in range(case.n):
        if chunk[i]:
            assert_close(got[case.cu[i]:case.cu[i + 1]], case.oracle_rows(i), dtype, f"seq {i}")
