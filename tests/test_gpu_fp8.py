"""GPU parity for the fp8 (E4M3, per-row scales) KV cache.

* kv_append: codes and scales bit for bit against the oracle's quantisation
  of the same bf16 rows (zero rows, tiny and large magnitudes, skipped slots,
  a NaN-filled pool around them);
* decode: the kernel's attention over the quantised cache against the
  oracle's attention over the same dequantised values (fp64), with the bf16
  tolerance, for every G and both head sizes, split-K included;
* the fused append + decode launch against append then decode, bit for bit;
* the quantisation error itself (fp8 cache against the unquantised bf16
  values) within its analytic bound.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import bf16 as OB
from oracle import quant as OQ
from tests.gpu_cases import FILL, assert_close, say

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _bf16(x):
    """fp32 values rounded to bf16 (as float32), the rows the cache is given."""
    return OB.round_bf16(np.asarray(x, np.float32)).astype(np.float32)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("Hkv,D", [(1, 64), (8, 128), (3, 64)])
def test_append_codes_and_scales_bitwise(kvc, Hkv, D):
    rng = np.random.default_rng(60 + D + Hkv)
    T, nb = 300, 40
    x = rng.standard_normal((2, T, Hkv, D)).astype(np.float32)
    x *= rng.choice([1e-6, 1e-3, 0.5, 3.0, 1e3], size=(2, T, Hkv, 1)).astype(np.float32)
    x[:, 7] = 0.0                                   # zero rows
    x[:, 8, :, 5] = 0.0
    x[0, 9, 0, :] = np.float32(2.0 ** -110)         # below the zero-row limit: stored as zeros
    x[1, 9, Hkv - 1, :2] = np.float32(2.0 ** -90)   # tiny but above it
    x = _bf16(x)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[[3, 50, 51]] = -1                         # skipped tokens
    say(f"fp8 append: {T} rows, Hkv {Hkv}, D {D}")
    cache = kvc.PagedKVCache.allocate(nb, Hkv, D, F8, fill_bits=FILL)
    kvc.kv_append(cache, torch.from_numpy(slots).cuda(), _dev(x[0]), _dev(x[1]))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    kc = cache.k_cache.view(torch.uint8).cpu().numpy()
    vc = cache.v_cache.view(torch.uint8).cpu().numpy()
    ks, vs = cache.k_scale.cpu().numpy(), cache.v_scale.cpu().numpy()
    written = np.zeros((nb * 16,), bool)
    for which, pool, sc in ((0, kc, ks), (1, vc, vs)):
        codes, scales = OQ.quantize_rows(x[which])
        for t in range(T):
            s = slots[t]
            if s < 0:
                continue
            written[s] = True
            assert np.array_equal(pool[s // 16, :, s % 16, :], codes[t]), (which, t)
            assert np.array_equal(sc[s // 16, :, s % 16].view(np.uint32),
                                  scales[t].view(np.uint32)), (which, t)
    # rows not written keep the sentinel
    for s in np.flatnonzero(~written)[:50]:
        assert np.all(kc[s // 16, :, s % 16, :] == 0xFF)
        assert np.all(np.isnan(ks[s // 16, :, s % 16]))


class Fp8Case:
    def __init__(self, wid, Hq, Hkv, D, ctx, seed_extra=0):
        self.w = W.small_workload(f"fp8-{wid}", wid, B=len(ctx), Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                                  sigma=0.5)
        self.ctx = np.asarray(ctx, np.int64)
        self.nb = int(sum(W.blocks_for(int(c)) for c in self.ctx)) + 5
        self.bt = W.block_tables(self.w, self.ctx, self.nb, seed_extra=seed_extra)
        self.vals = [W.sequence_values(self.w, b, int(n), 1) for b, n in enumerate(self.ctx)]
        # the bf16 rows the cache is given, and what the quantised cache holds
        self.kb = [_bf16(v[0]) for v in self.vals]
        self.vb = [_bf16(v[1]) for v in self.vals]
        self.qb = np.stack([_bf16(v[2][0]) for v in self.vals])
        self.kq = [OQ.dequantize_rows(*OQ.quantize_rows(k)) for k in self.kb]
        self.vq = [OQ.dequantize_rows(*OQ.quantize_rows(v)) for v in self.vb]

    def fill(self, kvc, upto_last=True):
        """Cache holding positions 0 .. ctx - 2 (or - 1 with upto_last)."""
        cache = kvc.PagedKVCache.allocate(self.nb, self.w.Hkv, self.w.D, F8, fill_bits=FILL)
        btd = torch.from_numpy(self.bt).cuda()
        n_of = [int(c) - (0 if upto_last else 1) for c in self.ctx]
        rows = [b for b in range(len(self.ctx)) if n_of[b] > 0]
        seq = np.concatenate([np.full(n_of[b], b, np.int32) for b in rows])
        pos = np.concatenate([np.arange(n_of[b], dtype=np.int32) for b in rows])
        s = kvc.slot_mapping(btd, self.nb, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                             err_flag=cache.err_flag)
        kvc.kv_append(cache, s, _dev(np.concatenate([self.kb[b][:n_of[b]] for b in rows])),
                      _dev(np.concatenate([self.vb[b][:n_of[b]] for b in rows])))
        return cache, btd

    def oracle(self, b, quantised=True):
        k = self.kq[b] if quantised else self.kb[b].astype(np.float64)
        v = self.vq[b] if quantised else self.vb[b].astype(np.float64)
        return OA.attend_row(self.qb[b].astype(np.float64), k, v, OA.default_scale(self.w.D))


CASES = [
    (32, 8, 128, [1, 2, 16, 17, 100, 2049, 5000]),     # G = 4, the serving shape
    (8, 8, 128, [3, 33, 700, 4100]),                    # G = 1
    (16, 8, 128, [20, 300, 1200]),                      # G = 2
    (64, 8, 128, [15, 640, 3000]),                      # G = 8
    (8, 2, 64, [1, 31, 2500, 257]),                     # G = 4, D 64
    (16, 2, 64, [9, 160, 6000]),                        # G = 8, D 64
]


@pytest.mark.parametrize("Hq,Hkv,D,ctx", CASES, ids=[f"{c[0]}/{c[1]}/{c[2]}" for c in CASES])
def test_decode_over_fp8_cache_matches_oracle(kvc, Hq, Hkv, D, ctx):
    case = Fp8Case(500 + Hq + D, Hq, Hkv, D, ctx)
    say(f"fp8 decode {Hq}/{Hkv}/{D}: ctx {ctx}")
    cache, btd = case.fill(kvc)
    out = kvc.paged_decode_attention(cache, _dev(case.qb), btd,
                                     torch.from_numpy(case.ctx.astype(np.int32)).cuda(),
                                     int(case.ctx.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    got = out.float().cpu().numpy()
    worst = 0.0
    for b in range(len(ctx)):
        worst = max(worst, assert_close(got[b], case.oracle(b), "bf16", f"fp8 decode row {b}"))
    say(f"  max abs err {worst:.2e}")


def _random_fp8_batches(seed, n):
    rng = np.random.default_rng(seed)
    lens = [1, 2, 15, 16, 17, 33, 257, 1000, 2049, 4100]
    return [(int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 8])),
             [int(x) for x in rng.choice(lens, size=int(rng.integers(1, 7)))]) for _ in range(n)]


FP8_SWEEP = _random_fp8_batches(78, 8)


@pytest.mark.parametrize("g,hkv,ctx", FP8_SWEEP, ids=[f"s{i}" for i in range(len(FP8_SWEEP))])
def test_random_batches_fp8_d128(kvc, g, hkv, ctx):
    """Seeded random batches through the fp8 block step at head dim 128 (the
    MFMA step): group sizes 1-8, 1-8 kv heads, contexts across block and
    partition boundaries; against the oracle over the dequantised cache."""
    i = FP8_SWEEP.index((g, hkv, ctx))
    case = Fp8Case(950 + i, g * hkv, hkv, 128, ctx, seed_extra=i)
    say(f"fp8 random batch {i}: G={g} Hkv={hkv} ctx {ctx}")
    cache, btd = case.fill(kvc)
    out = kvc.paged_decode_attention(cache, _dev(case.qb), btd,
                                     torch.from_numpy(case.ctx.astype(np.int32)).cuda(),
                                     int(case.ctx.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    got = out.float().cpu().numpy()
    for b in range(len(ctx)):
        assert_close(got[b], case.oracle(b), "bf16", f"fp8 random batch {i} row {b}")


def test_fused_append_decode_equals_append_then_decode(kvc):
    case = Fp8Case(560, 32, 8, 128, [1, 2, 16, 17, 31, 400, 3000, 2048], seed_extra=3)
    say("fp8 fused append + decode vs append then decode")
    ctx = torch.from_numpy(case.ctx.astype(np.int32)).cuda()
    mc = int(case.ctx.max())
    a, btd = case.fill(kvc, upto_last=False)
    k_new = _dev(np.stack([k[-1] for k in case.kb]))
    v_new = _dev(np.stack([v[-1] for v in case.vb]))
    out_fused = kvc.decode_append_attention(a, _dev(case.qb), k_new, v_new, btd, ctx, mc)
    b_cache, _ = case.fill(kvc, upto_last=True)
    out_ref = kvc.paged_decode_attention(b_cache, _dev(case.qb), btd, ctx, mc)
    torch.cuda.synchronize()
    assert torch.equal(out_fused.view(torch.int16), out_ref.view(torch.int16))
    assert torch.equal(a.k_cache.view(torch.uint8), b_cache.k_cache.view(torch.uint8))
    assert torch.equal(a.v_cache.view(torch.uint8), b_cache.v_cache.view(torch.uint8))
    used = torch.from_numpy(np.unique(case.bt[case.bt >= 0]).astype(np.int64)).cuda()
    for x, y in ((a.k_scale, b_cache.k_scale), (a.v_scale, b_cache.v_scale)):
        assert torch.equal(x.index_select(0, used).view(torch.int32),
                           y.index_select(0, used).view(torch.int32))
    got = out_fused.float().cpu().numpy()
    for b in range(len(case.ctx)):
        assert_close(got[b], case.oracle(b), "bf16", f"fused fp8 row {b}")


def test_quantisation_error_within_its_bound(kvc):
    """Attention over the fp8 cache against attention over the unquantised
    bf16 rows. Each dequantised value is within 1/16 of its magnitude (or
    2^-10 of its row scale below the normal range), so a logit moves by at
    most delta = scale * sum_d |q_d| err_k,d, the softmax weights by at most a
    factor exp(+-2 delta), and the output by at most
    max|v| (exp(2 delta) - 1) + max err_v; the kernel's own rounding adds the
    bf16 tolerance."""
    case = Fp8Case(570, 32, 8, 128, [50, 500, 2000, 6000])
    cache, btd = case.fill(kvc)
    out = kvc.paged_decode_attention(cache, _dev(case.qb), btd,
                                     torch.from_numpy(case.ctx.astype(np.int32)).cuda(),
                                     int(case.ctx.max()))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    scale = OA.default_scale(case.w.D)
    G = case.w.Hq // case.w.Hkv
    worst_rel = 0.0
    for b in range(len(case.ctx)):
        ref = case.oracle(b, quantised=False)
        kerr = np.abs(case.kq[b] - case.kb[b])          # [n, Hkv, D]
        verr = np.abs(case.vq[b] - case.vb[b])
        for hq in range(case.w.Hq):
            h = hq // G
            delta = scale * np.max(np.abs(case.qb[b, hq]) @ kerr[:, h, :].T)
            vmax = np.max(np.abs(case.vb[b][:, h, :]))
            bound = vmax * (np.exp(2 * delta) - 1) + np.max(verr[:, h, :]) + 1e-2
            err = np.max(np.abs(got[b, hq] - ref[hq]))
            assert err <= bound, (b, hq, err, bound)
            worst_rel = max(worst_rel, err / max(np.max(np.abs(ref[hq])), 1e-6))
    say(f"fp8 vs bf16 cache: worst error / max|out| = {worst_rel:.3e}")


def _random_fp8_prefill(seed, n):
    """Seeded head-dim-128 prefill shapes over an fp8 cache: group size, kv
    heads, prefixes and chunks on and beside the block and key-tile edges."""
    rng = np.random.default_rng(seed)
    pre, chk = [0, 1, 16, 63, 65, 500, 1700], [1, 16, 17, 64, 65, 200]
    out = []
    for _ in range(n):
        g, hkv, b = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3])), int(rng.integers(1, 4))
        out.append((g * hkv, hkv, 128, [int(x) for x in rng.choice(pre, size=b)],
                    [int(x) for x in rng.choice(chk, size=b)]))
    return out


PF_CASES = [
    (32, 8, 128, [0, 37, 300, 2000], [1, 17, 300, 200]),
    (8, 2, 64, [5, 100], [70, 9]),
    (16, 2, 64, [0, 3000], [130, 64]),
] + _random_fp8_prefill(83, 4)


@pytest.mark.parametrize("Hq,Hkv,D,prefix,chunk", PF_CASES,
                         ids=[f"{c[0]}/{c[1]}/{c[2]}-{i}" for i, c in enumerate(PF_CASES)])
@pytest.mark.parametrize("split", [False, True])
def test_chunked_prefill_over_fp8_cache(kvc, Hq, Hkv, D, prefix, chunk, split):
    """Prefill chunks written into an fp8 cache (quantised as kv_append does)
    and attended over the quantised prefix and chunk, against the oracle's
    attention over the same dequantised rows."""
    ctx = [p + c for p, c in zip(prefix, chunk)]
    w = W.small_workload(f"fp8-pf-{Hq}-{D}", 580 + Hq + D, B=len(ctx), Hq=Hq, Hkv=Hkv, D=D,
                         dtype="bf16", sigma=0.5)
    nb = int(sum(W.blocks_for(c) for c in ctx)) + 3
    bt = W.block_tables(w, np.array(ctx), nb)
    vals = [W.sequence_values(w, b, n, n) for b, n in enumerate(ctx)]
    kb = [_bf16(v[0]) for v in vals]
    vb = [_bf16(v[1]) for v in vals]
    qb = [_bf16(v[2]) for v in vals]
    say(f"fp8 prefill {Hq}/{Hkv}/{D} split={split}: prefix {prefix}, chunk {chunk}")
    cache = kvc.PagedKVCache.allocate(nb, Hkv, D, F8, fill_bits=FILL)
    btd = torch.from_numpy(bt).cuda()
    rows = [b for b in range(len(ctx)) if prefix[b] > 0]
    if rows:
        seq = np.concatenate([np.full(prefix[b], b, np.int32) for b in rows])
        pos = np.concatenate([np.arange(prefix[b], dtype=np.int32) for b in rows])
        s = kvc.slot_mapping(btd, nb, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                             err_flag=cache.err_flag)
        kvc.kv_append(cache, s, _dev(np.concatenate([kb[b][:prefix[b]] for b in rows])),
                      _dev(np.concatenate([vb[b][:prefix[b]] for b in rows])))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(chunk)]), dtype=torch.int32).cuda()
    q = _dev(np.concatenate([qb[b][prefix[b]:] for b in range(len(ctx))]))
    k = _dev(np.concatenate([kb[b][prefix[b]:] for b in range(len(ctx))]))
    v = _dev(np.concatenate([vb[b][prefix[b]:] for b in range(len(ctx))]))
    out = kvc.chunked_prefill_attention(cache, q, k, v, cu,
                                        torch.tensor(prefix, dtype=torch.int32).cuda(), btd,
                                        max(chunk), max_context_len=max(ctx) if split else None)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    got = out.float().cpu().numpy()
    scale = OA.default_scale(D)
    kc = cache.k_cache.view(torch.uint8).cpu().numpy()
    ksc = cache.k_scale.cpu().numpy()
    off, worst = 0, 0.0
    for b in range(len(ctx)):
        codes, scales = OQ.quantize_rows(kb[b])
        kq = OQ.dequantize_rows(codes, scales)
        vq = OQ.dequantize_rows(*OQ.quantize_rows(vb[b]))
        # the chunk's rows landed quantised, bit for bit
        for p in sorted({prefix[b], ctx[b] - 1, prefix[b] + chunk[b] // 2}):
            blk = bt[b, p // 16]
            assert np.array_equal(kc[blk, :, p % 16, :], codes[p]), (b, p)
            assert np.array_equal(ksc[blk, :, p % 16].view(np.uint32), scales[p].view(np.uint32))
        for r in range(chunk[b]):
            t = prefix[b] + r
            ref = OA.attend_row(qb[b][t].astype(np.float64), kq[:t + 1], vq[:t + 1], scale)
            worst = max(worst, assert_close(got[off + r], ref, "bf16", f"fp8 prefill {b} row {r}"))
        off += chunk[b]
    say(f"  max abs err {worst:.2e}")


_LONG = np.random.default_rng(5911).integers(1, 6000, 80).tolist()
MIXED_CASES = [
    (32, 8, 128, [1, 2, 17, 300, 2000, 5000], [0, 100, 3000], [33, 200, 64]),
    (16, 8, 128, [16, 33, 1000], [37], [300]),
    (8, 2, 64, [1, 65, 2500], [0, 250], [130, 17]),
    (32, 8, 128, _LONG, [2000], [300]),          # 640 decode items: rows ordered longest first
    (8, 8, 128, [1, 40, 1500, 4100], [0], [33]),  # G = 1 on the MFMA step's 16 head columns
]


@pytest.mark.parametrize("Hq,Hkv,D,dec_ctx,pf_prefix,pf_chunk", MIXED_CASES,
                         ids=["4-heads-mix", "g2", "d64", "80-rows", "g1"])
def test_mixed_step_over_fp8_cache(kvc, Hq, Hkv, D, dec_ctx, pf_prefix, pf_chunk):
    """The one-launch mixed step over an fp8 cache against the same step as
    separate calls (fused append + decode, then chunk write + prefill): the
    codes and scales it writes bit for bit, the prefill rows bit for bit (the
    same work item), and every decode row and sampled prefill rows against the
    oracle's attention over the dequantised rows, with the bf16 tolerance."""
    from tests.test_gpu_mixed import MixedCase
    case = MixedCase(f"fp8-mixed-{Hq}-{D}-{len(dec_ctx)}", 590 + Hq + D + len(dec_ctx), Hq, Hkv, D,
                     "bf16", dec_ctx, pf_prefix, pf_chunk)
    say(f"fp8 mixed step {Hq}/{Hkv}/{D}: {case.n_dec} decode rows, chunks {pf_chunk}")

    def fp8_fill():
        cache = kvc.PagedKVCache.allocate(case.nb, Hkv, D, F8, fill_bits=FILL)
        btd = torch.from_numpy(case.bt).cuda()
        rows = [b for b in range(len(case.ctx)) if case.cached_len(b) > 0]
        seq = np.concatenate([np.full(case.cached_len(b), b, np.int32) for b in rows])
        pos = np.concatenate([np.arange(case.cached_len(b), dtype=np.int32) for b in rows])
        s = kvc.slot_mapping(btd, case.nb, torch.from_numpy(seq).cuda(),
                             torch.from_numpy(pos).cuda(), err_flag=cache.err_flag)
        cached = lambda i: np.concatenate([case.vals[b][i][:case.cached_len(b)] for b in rows])
        kvc.kv_append(cache, s, _dev(cached(0)), _dev(cached(1)))
        return cache

    one, two = fp8_fill(), fp8_fill()
    inp = case.inputs()
    out_dec, out_pf = kvc.mixed_step_attention(one, Hq, **inp)
    ref_dec = kvc.decode_append_attention(two, inp["q_decode"], inp["k_new"], inp["v_new"],
                                          inp["decode_block_table"], inp["decode_context_lens"],
                                          inp["decode_max_context"])
    ref_pf = kvc.chunked_prefill_attention(two, inp["q_prefill"], inp["k_prefill"],
                                           inp["v_prefill"], inp["cu_chunk_lens"],
                                           inp["prefix_lens"], inp["prefill_block_table"],
                                           inp["prefill_max_chunk"])
    torch.cuda.synchronize()
    assert int(one.err_flag.item()) == 0 and int(two.err_flag.item()) == 0
    for x, y in ((one.k_cache, two.k_cache), (one.v_cache, two.v_cache)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    for x, y in ((one.k_scale, two.k_scale), (one.v_scale, two.v_scale)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(out_pf.view(torch.int16), ref_pf.view(torch.int16))

    scale = OA.default_scale(D)
    deq = lambda x: OQ.dequantize_rows(*OQ.quantize_rows(_bf16(x)))
    worst = 0.0
    got = out_dec.float().cpu().numpy()
    ref2 = ref_dec.float().cpu().numpy()
    for b in range(case.n_dec):
        c = case.dec_ctx[b]
        k, v, q = case.vals[b]
        ref = OA.attend_row(_bf16(q[c - 1]).astype(np.float64), deq(k[:c]), deq(v[:c]), scale)
        worst = max(worst, assert_close(got[b], ref, "bf16", f"fp8 mixed decode row {b} ctx {c}"))
        assert_close(got[b], ref2[b].astype(np.float64), "bf16", f"fp8 mixed vs separate, row {b}")
    got = out_pf.float().cpu().numpy()
    off = 0
    for i, (p0, C) in enumerate(zip(pf_prefix, pf_chunk)):
        k, v, q = case.vals[case.n_dec + i]
        kq, vq = deq(k[:p0 + C]), deq(v[:p0 + C])
        for r in sorted({0, C // 3, C - 1}):
            t = p0 + r
            ref = OA.attend_row(_bf16(q[t]).astype(np.float64), kq[:t + 1], vq[:t + 1], scale)
            worst = max(worst, assert_close(got[off + r], ref, "bf16",
                                            f"fp8 mixed chunk {i} row {r}"))
        off += C
    say(f"  max abs err {worst:.2e}")


def test_c3_full_size_fused_fp8(kvc):
    """The launch the fp8 bench line times, at its full size: the C3 batch (64
    sequences, contexts 2,000..2,300, GQA 32/8/128) over an fp8 cache, one
    fused quantising append + decode. Sampled rows (the shortest, the longest
    and six more) against the oracle over the dequantised rows, and their new
    rows' codes and scales bit for bit."""
    w = W.C3
    ctx = W.context_lengths(w)
    nb = W.C3_POOL_BLOCKS
    bt = W.block_tables(w, ctx, nb)
    vals = [W.sequence_values(w, b, int(n), 1) for b, n in enumerate(ctx)]
    say(f"fp8 C3 full size: {w.B} rows, sum ctx {int(ctx.sum())}, {nb} blocks")
    cache = kvc.PagedKVCache.allocate(nb, w.Hkv, w.D, F8, fill_bits=FILL)
    btd = torch.from_numpy(bt).cuda()
    seq = np.concatenate([np.full(int(n) - 1, b, np.int32) for b, n in enumerate(ctx)])
    pos = np.concatenate([np.arange(int(n) - 1, dtype=np.int32) for n in ctx])
    s = kvc.slot_mapping(btd, nb, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                         err_flag=cache.err_flag)
    kvc.kv_append(cache, s, _dev(np.concatenate([v[0][:-1] for v in vals])),
                  _dev(np.concatenate([v[1][:-1] for v in vals])))
    q = _dev(np.stack([v[2][0] for v in vals]))
    out = kvc.decode_append_attention(cache, q, _dev(np.stack([v[0][-1] for v in vals])),
                                      _dev(np.stack([v[1][-1] for v in vals])), btd,
                                      torch.from_numpy(ctx.astype(np.int32)).cuda(),
                                      int(ctx.max()))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    got = out.float().cpu().numpy()
    kc = cache.k_cache.view(torch.uint8).cpu().numpy()
    ksc = cache.k_scale.cpu().numpy()
    rng = np.random.default_rng(31)
    rows = sorted({int(np.argmin(ctx)), int(np.argmax(ctx))}
                  | set(rng.choice(w.B, 6, False).tolist()))
    scale = OA.default_scale(w.D)
    worst = 0.0
    for b in rows:
        kb, vb, qb = _bf16(vals[b][0]), _bf16(vals[b][1]), _bf16(vals[b][2][0])
        kcodes, kscales = OQ.quantize_rows(kb)
        kq = OQ.dequantize_rows(kcodes, kscales)
        vq = OQ.dequantize_rows(*OQ.quantize_rows(vb))
        p = int(ctx[b]) - 1                            # the row the fused launch wrote
        blk = bt[b, p // 16]
        assert np.array_equal(kc[blk, :, p % 16, :], kcodes[p]), b
        assert np.array_equal(ksc[blk, :, p % 16].view(np.uint32), kscales[p].view(np.uint32)), b
        ref = OA.attend_row(qb.astype(np.float64), kq, vq, scale)
        worst = max(worst, assert_close(got[b], ref, "bf16", f"fp8 C3 row {b} ctx {ctx[b]}"))
    say(f"  rows {rows}: max abs err {worst:.2e}")
