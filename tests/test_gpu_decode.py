"""GPU parity: append + paged decode attention against the oracle.

Tolerances: max-abs 1e-5 for fp32 caches and 1e-2 for bf16 caches against the
fp64 oracle on the same (bf16-rounded) values, plus a normalised bf16 bound
max|err| / max|ref| <= 2^-7, since at the Llama-shaped workload the outputs are
only about 0.01 in size.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import (FILL, TDTYPE, DecodeCase, assert_close, device_bits, oracle_values,
                             say, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _check_case(kvc, case: DecodeCase, check_pool=True, what="", fused=False):
    cache, out = case.run_gpu(kvc, fused=fused)
    assert int(cache.err_flag.item()) == 0
    if check_pool:
        pk, pv = case.oracle_pool()
        assert np.array_equal(device_bits(cache.k_cache), pk), f"{what}: K pool differs"
        assert np.array_equal(device_bits(cache.v_cache), pv), f"{what}: V pool differs"
    got = out.float().cpu().numpy()
    return assert_close(got, case.oracle_out(), case.w.dtype, what)


def test_c1_toy_generation_steps(kvc):
    """C1: a 16-token prompt cached, then 48 append+decode steps (context 17..64),
    each checked against the oracle's cached generation loop, which equals the
    recompute-everything loop bitwise."""
    w = W.C1
    n = W.C1_PROMPT + W.C1_ANSWER
    say("C1 toy fp32: 48 decode steps")
    k, v, q = W.sequence_values(w, 0, n, n)
    scale = OA.default_scale(w.D)
    ref_u, _, _ = OA.generate_uncached(q.astype(np.float64), k.astype(np.float64),
                                       v.astype(np.float64), W.C1_PROMPT, W.C1_ANSWER + 1, scale)
    bt = W.block_tables(w, np.array([n]), W.C1_POOL_BLOCKS)
    cache = kvc.PagedKVCache.allocate(W.C1_POOL_BLOCKS, w.Hkv, w.D, torch.float32, fill_bits=FILL)
    btd = torch.from_numpy(bt).cuda()
    z = lambda *a: torch.tensor(list(a), dtype=torch.int32, device="cuda")
    # prompt K/V into the cache
    s = kvc.slot_mapping(btd, W.C1_POOL_BLOCKS, z(*[0] * 16), z(*range(16)))
    kvc.kv_append(cache, s, to_device(k[:16], "fp32"), to_device(v[:16], "fp32"))
    outs = []
    for t in range(16, n):                      # 48 steps: context after append 17 .. 64
        s = kvc.slot_mapping(btd, W.C1_POOL_BLOCKS, z(0), z(t))
        kvc.kv_append(cache, s, to_device(k[t:t + 1], "fp32"), to_device(v[t:t + 1], "fp32"))
        o = kvc.paged_decode_attention(cache, to_device(q[t:t + 1], "fp32"), btd, z(t + 1), t + 1)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu().numpy()
    # uncached pass n+1 keeps row prompt+n-1; decode step at position t is pass t-14
    assert_close(got, ref_u[1:], "fp32", "C1 steps")
    assert int(cache.err_flag.item()) == 0


@pytest.mark.parametrize("ctx", [W.C2_CTX, W.C2_CTX + 1])
def test_c2_batch16(kvc, ctx):
    say(f"C2 batch 16 fp32 ctx={ctx}")
    case = DecodeCase(W.C2, np.full(W.C2.B, ctx), W.C2_POOL_BLOCKS + 16)
    _check_case(kvc, case, what=f"C2 ctx={ctx}")


@pytest.mark.parametrize("g", [1, 2, 4])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_grid_fp32_ctx_1_to_40(kvc, g, d):
    say(f"fp32 grid G={g} D={d} ctx 1..40")
    w = W.small_workload(f"grid-fp32-g{g}-d{d}", 100 + g * 1000 + d, B=40, Hq=2 * g, Hkv=2, D=d,
                         dtype="fp32")
    case = DecodeCase(w, np.arange(1, 41), 140)
    _check_case(kvc, case, what=f"fp32 G={g} D={d}")


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_grid_bf16(kvc, g, d):
    say(f"bf16 grid G={g} D={d}")
    w = W.small_workload(f"grid-bf16-g{g}-d{d}", 200 + g * 1000 + d, B=44, Hq=2 * g, Hkv=2, D=d,
                         dtype="bf16", sigma=0.5)
    ctx = np.concatenate([np.arange(1, 41), [100, 257, 300, 511]])
    case = DecodeCase(w, ctx, 200)
    _check_case(kvc, case, what=f"bf16 G={g} D={d}")


def test_split_k_long_contexts(kvc):
    say("split-K: bf16 32/8/128, ctx 5000, 3001, 17, 1")
    w = W.small_workload("splitk", 300, B=4, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    case = DecodeCase(w, [5000, 3001, 17, 1], 600)
    _check_case(kvc, case, what="split-K")


def test_c3_full_layer_bf16(kvc):
    say("C3 full layer bf16: B=64, ctx 2000..2300, 9,200-block pool")
    ctx = W.context_lengths(W.C3)
    case = DecodeCase(W.C3, ctx, W.C3_POOL_BLOCKS)
    _check_case(kvc, case, what="C3")


def test_c3_full_layer_bf16_fused(kvc):
    """The launch bench.py times: one fused append + decode per layer at C3."""
    say("C3 full layer bf16, fused append + decode launch")
    ctx = W.context_lengths(W.C3)
    case = DecodeCase(W.C3, ctx, W.C3_POOL_BLOCKS)
    _check_case(kvc, case, what="C3 fused", fused=True)


def test_c5_long_decode_fused(kvc):
    """C5 decode as its bench line times it: fused append + split-K decode + merge."""
    say("C5 decode: B=8, ctx 32,000, bf16, fused append + split-K")
    ctx = W.context_lengths(W.C5)
    case = DecodeCase(W.C5, ctx, 8 * W.blocks_for(W.C5_CTX))
    _check_case(kvc, case, check_pool=False, what="C5 decode fused", fused=True)


def test_c3_shape_fp32_cache(kvc):
    say("C3 shape with an fp32 cache at 1e-5")
    w = W.Workload("C3-fp32", 3, B=64, Hq=32, Hkv=8, D=128, dtype="fp32", sigma=0.5)
    case = DecodeCase(w, W.context_lengths(W.C3), W.C3_POOL_BLOCKS)
    _check_case(kvc, case, check_pool=False, what="C3 fp32")


def test_c5_long_decode(kvc):
    say("C5 decode: B=8, ctx 32,000, bf16, split-K")
    ctx = W.context_lengths(W.C5)
    case = DecodeCase(W.C5, ctx, 8 * W.blocks_for(W.C5_CTX))
    _check_case(kvc, case, check_pool=False, what="C5 decode")


def test_needle_through_block_table(kvc):
    """A key aligned with its query, 30+ logits above the rest, returns its value:
    pins the block-table indexing under bf16."""
    say("needle retrieval bf16")
    w = W.small_workload("needle", 400, B=6, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    ctx = np.array([2100, 900, 33, 16, 17, 4000])
    case = DecodeCase(w, ctx, 800)
    rng = np.random.default_rng(401)
    needles = []
    for b in range(w.B):
        j = int(rng.integers(0, ctx[b]))
        needles.append(j)
        for kh in range(w.Hkv):
            qh = case.q[b, kh * 4]
            case.q[b, kh * 4:(kh + 1) * 4] = qh               # the group's heads share the query
            qr = oracle_values(qh, "bf16")
            alpha = 60.0 * np.sqrt(w.D) / float(qr @ qr)
            case.k[b][j, kh] = alpha * qh
    cache, out = case.run_gpu(kvc)
    got = out.float().cpu().numpy()
    ref = case.oracle_out()
    assert_close(got, ref, "bf16", "needle")
    for b, j in enumerate(needles):                          # the oracle returns the needle's value
        vj = np.repeat(oracle_values(case.v[b][j], "bf16"), 4, axis=0)
        assert np.max(np.abs(ref[b] - vj)) < 1e-9
        assert np.max(np.abs(got[b] - vj)) <= 2.0 ** -8 * np.max(np.abs(vj))


def test_block_placement_does_not_change_results(kvc):
    say("two block permutations, same content: bitwise-equal outputs")
    w = W.small_workload("perm", 500, B=8, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    ctx = np.array([2000, 777, 16, 1, 300, 1500, 33, 64])
    a = DecodeCase(w, ctx, 400, seed_extra=0)
    b = DecodeCase(w, ctx, 400, seed_extra=1)
    assert not np.array_equal(a.bt, b.bt)
    _, oa = a.run_gpu(kvc)
    _, ob = b.run_gpu(kvc)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_context_zero_and_one(kvc):
    say("ctx 0 gives zeros, ctx 1 returns v exactly")
    for dtype in ("fp32", "bf16"):
        w = W.small_workload(f"ctx01-{dtype}", 600, B=3, Hq=8, Hkv=2, D=128, dtype=dtype)
        case = DecodeCase(w, [1, 0, 1], 8)
        cache, out = case.run_gpu(kvc, max_context_len=1)
        got = out.float().cpu().numpy()
        assert np.all(got[1] == 0)
        for b in (0, 2):
            want = np.repeat(oracle_values(case.v[b][0], dtype), 4, axis=0)
            assert np.array_equal(got[b], want)


def test_bad_block_id_is_flagged_not_faulted(kvc):
    say("block table with an id outside the pool")
    w = W.small_workload("badid", 700, B=2, Hq=8, Hkv=2, D=64, dtype="fp32")
    case = DecodeCase(w, [40, 40], 10)
    cache, _ = case.run_gpu(kvc)
    bt = torch.from_numpy(case.bt).cuda()
    bt[1, 1] = 10 ** 6
    q = to_device(case.q, "fp32")
    out = kvc.paged_decode_attention(cache, q, bt, torch.tensor([40, 40], dtype=torch.int32,
                                                                device="cuda"), 40)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & kvc.DEVERR_BLOCK_ID
    assert torch.isfinite(out).all()
    assert_close(out[0].cpu().numpy(), case.oracle_out([0])[0], "fp32", "row 0 unaffected")


@pytest.mark.parametrize("dtype,g,d", [("bf16", 4, 128), ("fp32", 1, 64), ("bf16", 8, 64),
                                       ("fp32", 2, 16)])
def test_fused_step_equals_separate_calls(kvc, dtype, g, d):
    """decode_append_attention == slot_mapping + kv_append + paged_decode_attention, bitwise,
    for the cache and for the outputs; and within tolerance of the oracle."""
    say(f"fused decode step vs separate calls {dtype} G={g} D={d}")
    w = W.small_workload(f"fused-{dtype}-{g}-{d}", 800 + g * 10 + d, B=7, Hq=2 * g, Hkv=2, D=d,
                         dtype=dtype, sigma=0.5)
    ctx = np.array([1, 16, 17, 300, 2500, 33, 64])
    case = DecodeCase(w, ctx, 320)
    cache_a, out_a = case.run_gpu(kvc)                      # separate calls
    # fused: same cache content before the step, then one launch
    cache_b = kvc.PagedKVCache.allocate(320, w.Hkv, w.D, TDTYPE[dtype], fill_bits=FILL)
    bt = torch.from_numpy(case.bt).cuda()
    old = [b for b in range(case.B) if ctx[b] > 1]
    seq = torch.from_numpy(np.concatenate([np.full(int(ctx[b]) - 1, b, np.int32) for b in old])).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(int(ctx[b]) - 1, dtype=np.int32) for b in old])).cuda()
    s = kvc.slot_mapping(bt, 320, seq, pos)
    kvc.kv_append(cache_b, s, to_device(np.concatenate([case.k[b][:-1] for b in old]), dtype),
                  to_device(np.concatenate([case.v[b][:-1] for b in old]), dtype))
    kn = to_device(np.stack([case.k[b][-1] for b in range(case.B)]), dtype)
    vn = to_device(np.stack([case.v[b][-1] for b in range(case.B)]), dtype)
    out_b = kvc.decode_append_attention(cache_b, to_device(case.q, dtype), kn, vn, bt,
                                        torch.from_numpy(ctx.astype(np.int32)).cuda(), int(ctx.max()))
    torch.cuda.synchronize()
    ib = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(cache_a.k_cache.view(ib), cache_b.k_cache.view(ib))
    assert torch.equal(cache_a.v_cache.view(ib), cache_b.v_cache.view(ib))
    assert torch.equal(out_a.view(ib), out_b.view(ib))
    assert int(cache_b.err_flag.item()) == 0
    assert_close(out_b.float().cpu().numpy(), case.oracle_out(), dtype, "fused")


def test_decode_at_140k_context_many_partitions(kvc):
    """A 140,000-token sequence beside a 1-token and a 70,001-token one, fused
    append + decode: the long ones split into many partitions (up to 256
    blocks each) whose partials the merge pass combines."""
    say("fused split-K decode at ctx 140,000 / 1 / 70,001, bf16 4/1/128")
    w = W.small_workload("splitk-140k", 310, B=3, Hq=4, Hkv=1, D=128, dtype="bf16", sigma=0.5)
    ctx = [140000, 1, 70001]
    case = DecodeCase(w, ctx, sum(W.blocks_for(c) for c in ctx) + 8)
    assert kvc.decode_workspace_bytes(3, 4, 128, 140000) > 0
    _check_case(kvc, case, what="split-K 140k", fused=True)


def _random_batches(seed, n):
    """Seeded batch shapes: group size, kv heads, contexts (at block, partition
    and ragged boundaries), plain or fused."""
    rng = np.random.default_rng(seed)
    lens = [1, 2, 15, 16, 17, 31, 33, 255, 257, 1000, 2049, 4100]
    out = []
    for _ in range(n):
        g, hkv, b = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3, 8])), int(rng.integers(1, 9))
        out.append((g, hkv, [int(x) for x in rng.choice(lens, size=b)], bool(rng.integers(0, 2))))
    return out


SWEEP = _random_batches(73, 12)


@pytest.mark.parametrize("g,hkv,ctx,fused", SWEEP, ids=[f"s{i}" for i in range(len(SWEEP))])
def test_random_batches_bf16_d128(kvc, g, hkv, ctx, fused):
    """Seeded random batches through the bf16 block step at head dim 128 (the
    MFMA step of the decode kernel): group sizes 1-8, 1-8 kv heads, 1-8 rows
    whose contexts cross block and partition boundaries, plain and fused;
    against the oracle, and the pool bit for bit."""
    i = SWEEP.index((g, hkv, ctx, fused))
    say(f"random batch {i}: G={g} Hkv={hkv} ctx {ctx} fused {fused}")
    w = W.small_workload(f"sweep-{i}", 900 + i, B=len(ctx), Hq=g * hkv, Hkv=hkv, D=128, dtype="bf16",
                         sigma=0.5)
    case = DecodeCase(w, ctx, sum(W.blocks_for(c) for c in ctx) + 8, seed_extra=i)
    _check_case(kvc, case, what=f"random batch {i}", fused=fused)


def test_split_k_agrees_with_one_partition(kvc):
    """The same 3,000-token sequence decoded as row 0 of a 64-row batch (one
    partition: the batch already fills 512 workgroups) and alone (3
    partitions of 64 blocks and the merge): each within the oracle's tolerance, and within
    it of each other."""
    say("split-K vs one partition, fp32 32/8/128, ctx 3,000")
    w = W.small_workload("split-vs-one", 320, B=64, Hq=32, Hkv=8, D=128, dtype="fp32")
    ctx = [3000] + [300] * 63
    batch = DecodeCase(w, ctx, sum(W.blocks_for(c) for c in ctx) + 8)
    alone = DecodeCase(w, [3000], W.blocks_for(3000) + 8)     # row 0's values, same seed
    assert np.array_equal(alone.q[0], batch.q[0])
    _, ob = batch.run_gpu(kvc)
    _, oa = alone.run_gpu(kvc)
    ref = alone.oracle_out()
    got_b, got_a = ob.float().cpu().numpy()[:1], oa.float().cpu().numpy()
    assert_close(got_b, ref, "fp32", "one partition")
    assert_close(got_a, ref, "fp32", "3 partitions")
    assert_close(got_a, got_b, "fp32", "split vs one partition")


def test_gqa_equals_mha_over_repeated_heads(kvc):
    """Grouped-query attention is multi-head attention with each K/V head
    repeated G times: the G = 4 decode over 2 kv heads and the G = 1 decode over
    the 8 heads made by repeating them agree (fp32)."""
    say("GQA 8/2 vs MHA 8/8 over repeated K/V heads, fp32 D=64")
    wg = W.small_workload("gqa-vs-mha", 330, B=4, Hq=8, Hkv=2, D=64, dtype="fp32")
    wm = W.small_workload("gqa-vs-mha-rep", 331, B=4, Hq=8, Hkv=8, D=64, dtype="fp32")
    ctx = [1, 17, 300, 1000]
    g = DecodeCase(wg, ctx, 200)
    m = DecodeCase(wm, ctx, 200)
    m.q = g.q.copy()
    m.k = [np.repeat(k, 4, axis=1) for k in g.k]
    m.v = [np.repeat(v, 4, axis=1) for v in g.v]
    _, og = g.run_gpu(kvc)
    _, om = m.run_gpu(kvc)
    got_g, got_m = og.float().cpu().numpy(), om.float().cpu().numpy()
    assert_close(got_g, g.oracle_out(), "fp32", "GQA")
    assert_close(got_m, got_g, "fp32", "MHA over repeated heads vs GQA")
