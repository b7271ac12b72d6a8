"""GPU: kvc_decode_append_attention_noalloc, the fused decode step whose
split-K partials live in the library's per-device scratch array.

Two calls in a row (the second smaller), each split over several partitions
so the scratch array is really used, each compared with
kvc_decode_append_attention (same kernels, caller workspace) on an identical
cache: outputs and pools bit for bit, and the outputs against the oracle
within the bf16 tolerance. A call that would need more than KVC_SCRATCH_BYTES
is rejected with KVC_ERR_SCRATCH before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_cases import DecodeCase, assert_close, device_bits, say, to_device

pytestmark = pytest.mark.gpu
KVC_ERR_SCRATCH = -11
SCRATCH_BYTES = 16 << 20


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _cache_before_step(kvc, case):
    """A NaN pool holding positions 0 .. ctx - 2 of every row."""
    w = case.w
    cache = kvc.PagedKVCache.allocate(case.num_blocks, w.Hkv, w.D, torch.bfloat16, fill_bits=-1)
    bt = torch.from_numpy(case.bt).cuda()
    seq = np.concatenate([np.full(int(n) - 1, b, np.int32) for b, n in enumerate(case.ctx)])
    pos = np.concatenate([np.arange(int(n) - 1, dtype=np.int32) for n in case.ctx])
    s = kvc.slot_mapping(bt, case.num_blocks, torch.from_numpy(seq).cuda(),
                         torch.from_numpy(pos).cuda(), err_flag=cache.err_flag)
    kvc.kv_append(cache, s, to_device(np.concatenate([k[:-1] for k in case.k]), "bf16"),
                  to_device(np.concatenate([v[:-1] for v in case.v]), "bf16"))
    return cache, bt


@pytest.mark.parametrize("ctx_pair", [([9000, 20000, 5000, 33], [3000, 700])])
def test_noalloc_equals_workspace_call_twice(kvc, ctx_pair):
    for call, ctx in enumerate(ctx_pair):
        ctx = np.asarray(ctx)
        w = W.small_workload(f"noalloc-{call}", 9300 + call, B=len(ctx), Hq=32, Hkv=8, D=128,
                             dtype="bf16", sigma=0.5)
        nb = int(sum(W.blocks_for(int(c)) for c in ctx)) + 3
        case = DecodeCase(w, ctx, nb)
        mcl = int(ctx.max())
        need = kvc.decode_workspace_bytes(case.B, w.Hq, w.D, mcl)
        say(f"noalloc call {call}: B={case.B} ctx={ctx.tolist()} (workspace rule {need} B)")
        assert need > 0, "the case must split so that the scratch array is used"
        q = to_device(case.q, "bf16")
        kn = to_device(np.stack([k[-1] for k in case.k]), "bf16")
        vn = to_device(np.stack([v[-1] for v in case.v]), "bf16")
        lens = torch.from_numpy(ctx.astype(np.int32)).cuda()

        ref_cache, bt = _cache_before_step(kvc, case)
        ref = kvc.decode_append_attention(ref_cache, q, kn, vn, bt, lens, mcl)
        cache, _ = _cache_before_step(kvc, case)
        out = torch.empty_like(q)
        got = kvc.decode_append_attention_noalloc(cache, q, kn, vn, bt, lens, mcl, out)
        torch.cuda.synchronize()
        assert got is out
        assert int(cache.err_flag.item()) == 0 and int(ref_cache.err_flag.item()) == 0
        assert np.array_equal(device_bits(out), device_bits(ref)), f"call {call}: outputs differ"
        assert np.array_equal(device_bits(cache.k_cache), device_bits(ref_cache.k_cache))
        assert np.array_equal(device_bits(cache.v_cache), device_bits(ref_cache.v_cache))
        assert_close(out.float().cpu().numpy(), case.oracle_out(), "bf16", f"noalloc call {call}")


def test_noalloc_rejects_a_call_past_the_scratch_size(kvc):
    """256 rows x 32 heads at a 65,536-token bound split 16 ways: 68 MB of
    partials, more than the 16 MiB array; rejected before any launch."""
    B, Hq, Hkv, D, mcl = 256, 32, 8, 128, 65536
    assert B * Hq * 16 * (4 * D + 8) > SCRATCH_BYTES
    say("noalloc: a call past the scratch size is rejected")
    cache = kvc.PagedKVCache.allocate(16, Hkv, D, torch.bfloat16, fill_bits=0)
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(B, Hkv, D, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, mcl // 16, dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    st = kvc.LIB.kvc_decode_append_attention_noalloc(
        cache.c, q.data_ptr(), kn.data_ptr(), kn.data_ptr(), B, Hq, bt.data_ptr(), bt.shape[1],
        lens.data_ptr(), mcl, 0.1, out.data_ptr(), None)
    assert st == KVC_ERR_SCRATCH
    assert b"scratch" in kvc.LIB.kvc_status_string(st)
    with pytest.raises(kvc.KvcError):
        kvc.decode_append_attention_noalloc(cache, q, kn, kn, bt, lens, mcl, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "nothing was launched"
