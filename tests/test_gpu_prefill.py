"""GPU parity: chunked-prefill attention (MFMA) and its chunk K/V write."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_cases import PrefillCase, assert_close, device_bits, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _check(kvc, case: PrefillCase, what: str, pool=True, rows=None, max_context_len=None):
    cache, out = case.run_gpu(kvc, max_context_len=max_context_len)
    assert int(cache.err_flag.item()) == 0
    if pool:
        pk, pv = case.oracle_pool()
        assert np.array_equal(device_bits(cache.k_cache), pk), f"{what}: K pool differs"
        assert np.array_equal(device_bits(cache.v_cache), pv), f"{what}: V pool differs"
    got = out.float().cpu().numpy()
    for i in range(case.n):
        g = got[case.cu[i]:case.cu[i + 1]]
        if rows is None:
            assert_close(g, case.oracle_rows(i), case.w.dtype, f"{what} seq {i}")
        else:
            r = rows(i)
            assert_close(g[r], case.oracle_rows(i, r), case.w.dtype, f"{what} seq {i}")
    return cache, out


def test_c1_prompt_prefill(kvc):
    """C1's 16-token prompt (prefix 0), fp32, MHA 4/4, head_dim 16."""
    say("prefill C1 prompt fp32")
    case = PrefillCase(W.C1, [0], [W.C1_PROMPT], W.C1_POOL_BLOCKS)
    _check(kvc, case, "C1 prefill")


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype,d", [("fp32", 16), ("fp32", 64), ("fp32", 128), ("bf16", 32),
                                     ("bf16", 64), ("bf16", 128)])
def test_ragged_batch(kvc, dtype, d, g):
    say(f"prefill ragged batch {dtype} D={d} G={g}")
    w = W.small_workload(f"pf-{dtype}-{d}-{g}", 900 + g * 1000 + d, B=6, Hq=2 * g, Hkv=2, D=d,
                         dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0)
    prefix = [0, 17, 100, 31, 64, 0]
    chunk = [1, 16, 33, 200, 64, 130]
    case = PrefillCase(w, prefix, chunk, 120)
    _check(kvc, case, f"{dtype} D={d} G={g}")


def test_chunked_equals_one_shot_bf16(kvc):
    """Prefill in chunks [0,100), [100,257), [257,300) gives the same cache bits
    and, within tolerance, the same rows as one 300-token prefill."""
    say("prefill chunked vs one-shot bf16 32/8/128")
    w = W.small_workload("pf-chunks", 950, B=1, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    one = PrefillCase(w, [0], [300], 40)
    c1, o1 = one.run_gpu(kvc)
    ref = one.oracle_rows(0)
    assert_close(o1.float().cpu().numpy(), ref, "bf16", "one-shot")
    cache = kvc.PagedKVCache.allocate(40, w.Hkv, w.D, torch.bfloat16, fill_bits=-1)
    outs = []
    from tests.gpu_cases import to_device
    dev = "cuda"
    for a, b in [(0, 100), (100, 257), (257, 300)]:
        # each call writes only its chunk; earlier chunks are already cached
        cu = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        out = kvc.chunked_prefill_attention(
            cache, to_device(one.q[0][a:b], "bf16"), to_device(one.k[0][a:b], "bf16"),
            to_device(one.v[0][a:b], "bf16"), cu, torch.tensor([a], dtype=torch.int32, device=dev),
            torch.from_numpy(one.bt).to(dev), b - a)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(cache.k_cache.view(torch.int16), c1.k_cache.view(torch.int16))
    assert torch.equal(cache.v_cache.view(torch.int16), c1.v_cache.view(torch.int16))
    assert_close(torch.cat(outs).float().cpu().numpy(), ref, "bf16", "chunked")


def test_one_token_chunk_matches_decode(kvc):
    say("prefill with C = 1 vs decode of the same position")
    w = W.small_workload("pf-c1", 960, B=3, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    case = PrefillCase(w, [2100, 15, 0], [1, 1, 1], 200)
    cache, out = case.run_gpu(kvc)
    bt = torch.from_numpy(case.bt).cuda()
    ctx = torch.from_numpy(case.total.astype(np.int32)).cuda()
    from tests.gpu_cases import to_device
    dec = kvc.paged_decode_attention(cache, to_device(np.concatenate(case.q), "bf16"), bt, ctx,
                                     int(case.total.max()))
    torch.cuda.synchronize()
    ref = np.concatenate([case.oracle_rows(i) for i in range(3)])
    assert_close(out.float().cpu().numpy(), ref, "bf16", "prefill C=1")
    assert_close(dec.float().cpu().numpy(), ref, "bf16", "decode")


def test_c5_prefill_chunk_over_long_prefix(kvc):
    """C5: 8 sequences x a 2,048-token chunk over a 30,000-token cached prefix.
    Rows sampled per sequence (first, last, block edges and seeded random)."""
    say("prefill C5: 8 x 2048 over 30,000 prefix, bf16, sampled rows")
    n = W.C5.B
    case = PrefillCase(W.C5, [W.C5_PREFIX] * n, [W.C5_CHUNK] * n,
                       n * W.blocks_for(W.C5_PREFIX + W.C5_CHUNK))
    rng = np.random.default_rng(961)

    def rows(i):
        return sorted(set([0, 1, 15, 16, 1023, 2047] + rng.integers(0, W.C5_CHUNK, 4).tolist()))
    cache, out = _check(kvc, case, "C5 prefill", pool=False, rows=rows)
    # every row and head of sequence 0's first and last query tile (the last holds
    # the causal diagonal), against the matrix-form oracle
    from oracle import attention as OA
    from tests.gpu_cases import oracle_values
    mp = 256 // (W.C5.Hq // W.C5.Hkv)               # positions per query tile
    got = out.float().cpu().numpy()[case.cu[0]:case.cu[1]]
    kq, vq = oracle_values(case.k[0], "bf16"), oracle_values(case.v[0], "bf16")
    for lo in (0, W.C5_CHUNK - mp):
        r = np.arange(lo, lo + mp)
        ref = OA.attend_positions(oracle_values(case.q[0][r], "bf16"), kq, vq, W.C5_PREFIX + r,
                                  OA.default_scale(W.C5.D))
        assert_close(got[r], ref, "bf16", f"C5 seq 0 query tile at {lo}, every row and head")
    # the chunk's K/V landed at their slots (sampled tokens, bitwise)
    from oracle import paged as OP
    from tests.gpu_cases import oracle_bits
    kb = device_bits(cache.k_cache)
    for i in range(n):
        for p in [W.C5_PREFIX, W.C5_PREFIX + 1, W.C5_PREFIX + 2047]:
            s = OP.slot_of(case.bt[i], p, 16)
            assert np.array_equal(kb[s // 16, :, s % 16, :], oracle_bits(case.k[i][p], "bf16"))


@pytest.mark.parametrize("dtype,d,g", [("bf16", 128, 4), ("bf16", 64, 8), ("bf16", 32, 1),
                                       ("fp32", 64, 2), ("fp32", 128, 4)])
def test_split_keys_short_chunks_over_long_prefixes(kvc, dtype, d, g):
    """Few query tiles over long prefixes: the split entry point spreads each
    query tile's keys over several workgroups and merges them. The 700-token
    chunk over no prefix has query tiles whose keys end before the later
    splits start (empty partials)."""
    w = W.small_workload(f"pf-split-{dtype}-{d}-{g}", 970 + g * 100 + d, B=4, Hq=2 * g, Hkv=2,
                         D=d, dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0)
    prefix = [1900, 3000, 0, 257]
    chunk = [100, 7, 700, 64]
    max_ctx = max(p + c for p, c in zip(prefix, chunk))
    need = kvc.prefill_workspace_bytes(4, sum(chunk), max(chunk), max_ctx, w.Hq, w.Hkv, d)
    assert need > 0, "this case is meant to split"
    say(f"prefill split {dtype} D={d} G={g}: workspace {need} B")
    case = PrefillCase(w, prefix, chunk, 400)
    _check(kvc, case, f"split {dtype} D={d} G={g}", max_context_len=max_ctx)


def _random_prefill_batches(seed, n):
    """Seeded batch shapes for the MFMA prefill at head dim 128: group size, kv
    heads, prefix and chunk lengths on and beside the 16-token block and the
    64-key tile boundaries (prefixes long enough for the key-range split to
    cut), through the plain or the split entry point."""
    rng = np.random.default_rng(seed)
    pre = [0, 1, 15, 16, 63, 64, 65, 255, 700, 1500, 2600]
    chk = [1, 2, 16, 17, 63, 64, 65, 129, 256, 300]
    out = []
    for _ in range(n):
        g, hkv, b = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3])), int(rng.integers(1, 5))
        out.append((g, hkv, [int(x) for x in rng.choice(pre, size=b)],
                    [int(x) for x in rng.choice(chk, size=b)], bool(rng.integers(0, 2))))
    return out


PF_SWEEP = _random_prefill_batches(91, 10)


@pytest.mark.parametrize("g,hkv,prefix,chunk,split", PF_SWEEP, ids=[f"p{i}" for i in range(len(PF_SWEEP))])
def test_random_batches_bf16_d128(kvc, g, hkv, prefix, chunk, split):
    """Seeded random batches through the bf16 prefill at head dim 128 (the
    two-group MFMA pipeline): every row against the oracle, the pool bit for
    bit."""
    i = PF_SWEEP.index((g, hkv, prefix, chunk, split))
    total = [p + c for p, c in zip(prefix, chunk)]
    say(f"random prefill {i}: G={g} Hkv={hkv} prefix {prefix} chunk {chunk} split {split}")
    w = W.small_workload(f"pf-sweep-{i}", 3100 + i, B=len(prefix), Hq=g * hkv, Hkv=hkv, D=128,
                         dtype="bf16", sigma=0.5)
    case = PrefillCase(w, prefix, chunk, sum(W.blocks_for(t) for t in total) + 4, seed_extra=i)
    _check(kvc, case, f"random prefill {i}", max_context_len=max(total) if split else None)


def test_split_entry_without_split_is_the_same_kernel(kvc):
    """C5-sized work needs no split: the split entry point gives the plain call's bits."""
    say("prefill split entry, no split needed: bitwise equal to the plain call")
    w = W.small_workload("pf-nosplit", 985, B=8, Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    case = PrefillCase(w, [500] * 8, [512] * 8, 8 * 64)
    assert kvc.prefill_workspace_bytes(8, 8 * 512, 512, 1012, 32, 8, 128) == 0
    _, plain = case.run_gpu(kvc)
    _, split = case.run_gpu(kvc, max_context_len=1012)
    assert torch.equal(plain, split)


def test_split_context_bound_too_small_is_flagged(kvc):
    """A sequence longer than max_context_len: the rows miss keys, and the
    device flag says so (no access outside the pool either way)."""
    say("prefill split with max_context_len below a sequence's length")
    w = W.small_workload("pf-split-bad", 986, B=1, Hq=8, Hkv=2, D=64, dtype="bf16", sigma=0.5)
    case = PrefillCase(w, [3000], [7], 300)
    cache, _ = case.run_gpu(kvc, max_context_len=1000)
    assert int(cache.err_flag.item()) & kvc.DEVERR_CONTEXT


@pytest.mark.parametrize("dtype,d,g", [("bf16", 128, 4), ("bf16", 64, 2), ("fp32", 64, 1)])
def test_bad_prefix_block_id_is_flagged_not_faulted(kvc, dtype, d, g):
    """A block id outside the pool in a prefix's table: the kernel reads no key
    from it (zeros instead), flags the contract violation and writes finite rows.
    Covers the buffer->LDS staging (bf16) and the register staging (fp32)."""
    say(f"prefill with a bad prefix block id, {dtype} D={d} G={g}")
    w = W.small_workload(f"pf-badblk-{dtype}", 987 + d + g, B=2, Hq=2 * g, Hkv=2, D=d, dtype=dtype,
                         sigma=0.5 if dtype == "bf16" else 1.0)
    case = PrefillCase(w, [100, 200], [40, 70], 64)
    cache, _ = case.run_gpu(kvc)
    assert int(cache.err_flag.item()) == 0
    bad = case.bt.copy()
    bad[1, 3] = case.num_blocks + 7                    # keys 48..63 of sequence 1's prefix
    q = to_device(np.concatenate(case.q), w.dtype)
    k = to_device(np.concatenate([case.k[i][case.prefix[i]:] for i in range(case.n)]), w.dtype)
    v = to_device(np.concatenate([case.v[i][case.prefix[i]:] for i in range(case.n)]), w.dtype)
    out = kvc.chunked_prefill_attention(
        cache, q, k, v, torch.from_numpy(case.cu).cuda(),
        torch.from_numpy(case.prefix.astype(np.int32)).cuda(), torch.from_numpy(bad).cuda(),
        int(case.chunk.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & kvc.DEVERR_BLOCK_ID
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    # sequence 0's table is intact: its rows are still right
    assert_close(got[case.cu[0]:case.cu[1]], case.oracle_rows(0), dtype, "intact sequence 0")


@pytest.mark.parametrize("dtype,d,g,prefix,chunk", [("fp32", 128, 1, 40000, 48),
                                                    ("bf16", 64, 2, 140000, 37),
                                                    ("bf16", 128, 4, 140000, 21)])
def test_prefix_past_the_block_row_cache(kvc, dtype, d, g, prefix, chunk):
    """The workgroup keeps the pool rows of its first blocks in LDS (8,192
    blocks with buffer->LDS staging, 2,048 with register staging); keys past
    them look their block up in the table directly. A chunk over a prefix of
    40,000 (fp32, register staging) or 140,000 (bf16) keys crosses that edge."""
    say(f"prefill over a {prefix}-key prefix, {dtype} D={d} G={g}, chunk {chunk}")
    w = W.small_workload(f"pf-long-{dtype}-{d}-{g}", 990 + d + g, B=1, Hq=g, Hkv=1, D=d,
                         dtype=dtype, sigma=0.5 if dtype == "bf16" else 1.0)
    case = PrefillCase(w, [prefix], [chunk], W.blocks_for(prefix + chunk) + 16)
    _check(kvc, case, f"long prefix {dtype} D={d}", pool=False)
