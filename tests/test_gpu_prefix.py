"""GPU parity for prefix caching: a prompt sharing its first 1,800 tokens with
a cached 2,000-token prompt (daviddominguez.dev, section "A prefix already in
the cache can skip its prefill") reuses the cached blocks found by the native
block manager and prefills only the rest. The warm prefill must equal a cold
prefill of the same prompt into unshared blocks bit for bit, agree with the
oracle, leave the shared blocks untouched, and decode over the shared blocks
must equal decode over the unshared copy bit for bit.

Values depend on the whole token prefix (workloads.prefix_values), so the
shared opening holds the same keys and values in both prompts.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle.prefix import PrefixCache as OraclePrefix
from tests.gpu_cases import assert_close, device_bits, oracle_values, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _prefill(kvc, cache, q, k, v, prefix, blocks, max_blocks):
    dev = cache.k_cache.device
    C = q.shape[0]
    bt = torch.full((1, max_blocks), -1, dtype=torch.int32)
    bt[0, :len(blocks)] = torch.tensor(blocks, dtype=torch.int32)
    cu = torch.tensor([0, C], dtype=torch.int32, device=dev)
    pre = torch.tensor([prefix], dtype=torch.int32, device=dev)
    return kvc.chunked_prefill_attention(cache, to_device(q, "bf16"), to_device(k, "bf16"),
                                         to_device(v, "bf16"), cu, pre, bt.to(dev), C)


def _decode(kvc, cache, q, k, v, ctx, blocks, max_blocks):
    dev = cache.k_cache.device
    bt = torch.full((1, max_blocks), -1, dtype=torch.int32)
    bt[0, :len(blocks)] = torch.tensor(blocks, dtype=torch.int32)
    ctx_t = torch.tensor([ctx], dtype=torch.int32, device=dev)
    return kvc.decode_append_attention(cache, to_device(q[None], "bf16"), to_device(k[None], "bf16"),
                                       to_device(v[None], "bf16"), bt.to(dev), ctx_t, ctx)


def test_warm_prefill_over_shared_blocks(kvc):
    w = W.P1
    A, B = W.shared_prompts(2)
    n = len(A)
    say(f"prefix caching: prompts of {n} tokens sharing {W.P1_SHARED}")
    kA, vA, qA = W.prefix_values(w, A)
    extra = 12345
    kB, vB, qB = W.prefix_values(w, B + [extra])     # position n is the decode token
    nb, maxb = 400, 130
    pc = kvc.PrefixCache(nb)
    orc = OraclePrefix(nb)
    cache = kvc.PagedKVCache.allocate(nb, w.Hkv, w.D, torch.bfloat16, fill_bits=-1)

    # request A, cold: every block fresh, committed once written
    ba = pc.allocate(W.blocks_for(n))
    assert ba == orc.allocate(W.blocks_for(n))
    _prefill(kvc, cache, qA, kA, vA, 0, ba, maxb)
    pc.commit(A, ba)
    orc.commit(A, ba)
    torch.cuda.synchronize()
    shared_bits = device_bits(cache.k_cache[ba[:112]]), device_bits(cache.v_cache[ba[:112]])

    # request B, warm: 112 whole blocks (1,792 tokens) matched, 208 tokens prefilled
    m = pc.match(B)
    assert m == orc.match(B) == ba[:112]
    start = 16 * len(m)
    fresh = pc.allocate(W.blocks_for(n) - len(m))
    assert fresh == orc.allocate(W.blocks_for(n) - len(m))
    bb = m + fresh
    out_warm = _prefill(kvc, cache, qB[start:n], kB[start:n], vB[start:n], start, bb, maxb)

    # request B again, cold, into blocks nobody shares
    bc = pc.allocate(W.blocks_for(n))
    out_cold = _prefill(kvc, cache, qB[:n], kB[:n], vB[:n], 0, bc, maxb)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0

    assert torch.equal(out_warm, out_cold[start:]), "warm prefill differs from cold"
    # the shared blocks were read, not written
    assert np.array_equal(device_bits(cache.k_cache[ba[:112]]), shared_bits[0])
    assert np.array_equal(device_bits(cache.v_cache[ba[:112]]), shared_bits[1])
    assert [pc.refcount(b) for b in ba[:112]] == [2] * 112
    assert [pc.refcount(b) for b in ba[112:]] == [1] * (len(ba) - 112)

    scale = OA.default_scale(w.D)
    got = out_warm.float().cpu().numpy()
    for r in [0, 1, 15, 16, 100, n - start - 1]:
        p = start + r
        ref = OA.attend_row(oracle_values(qB[p], "bf16"), oracle_values(kB[:p + 1], "bf16"),
                            oracle_values(vB[:p + 1], "bf16"), scale)
        assert_close(got[r], ref, "bf16", f"warm prefill row {p}")

    # the same warm prefill through the key-range split (8 splits of 4 tiles)
    out_split = kvc.chunked_prefill_attention(
        cache, to_device(qB[start:n], "bf16"), to_device(kB[start:n], "bf16"),
        to_device(vB[start:n], "bf16"), torch.tensor([0, n - start], dtype=torch.int32).cuda(),
        torch.tensor([start], dtype=torch.int32).cuda(),
        torch.tensor([bb + [-1] * (maxb - len(bb))], dtype=torch.int32).cuda(), n - start,
        max_context_len=n)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    got_s = out_split.float().cpu().numpy()
    assert_close(got_s, out_warm.float().cpu().numpy(), "bf16", "split vs unsplit warm prefill")
    for r in [0, 100, n - start - 1]:
        p = start + r
        ref = OA.attend_row(oracle_values(qB[p], "bf16"), oracle_values(kB[:p + 1], "bf16"),
                            oracle_values(vB[:p + 1], "bf16"), scale)
        assert_close(got_s[r], ref, "bf16", f"split warm prefill row {p}")

    # one decode step of B over the shared blocks and over the unshared copy
    more = pc.allocate(2)
    d_shared = _decode(kvc, cache, qB[n], kB[n], vB[n], n + 1, bb + more[:1], maxb)
    d_copy = _decode(kvc, cache, qB[n], kB[n], vB[n], n + 1, bc + more[1:], maxb)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    assert torch.equal(d_shared, d_copy), "decode over shared blocks differs"
    ref = OA.attend_row(oracle_values(qB[n], "bf16"), oracle_values(kB[:n + 1], "bf16"),
                        oracle_values(vB[:n + 1], "bf16"), scale)
    assert_close(d_shared.float().cpu().numpy()[0], ref, "bf16", "decode after warm prefill")

    pc.release(bb + more[:1])
    pc.release(bc + more[1:])
    pc.release(ba)
    assert pc.counts() == (nb - 125, 125, 0)
