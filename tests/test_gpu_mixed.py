"""GPU parity for the one-launch mixed step (kvc_mixed_step_attention): decode
rows and prefill chunks of one continuous-batching step in a single persistent
kernel. Every output row is checked against the oracle's attention, the cache
afterwards against the inputs bit for bit, the prefill rows bit for bit against
kvc_chunked_prefill_attention, and the workspace header is zero again after
each call (calls share one workspace).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import paged as OP
from tests.gpu_cases import (FILL, TDTYPE, assert_close, device_bits, oracle_bits, oracle_values,
                             say, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


class MixedCase:
    """Decode rows (ctx counts the new token) and prefill chunks (prefix,
    chunk) over one pool; every sequence's values are seeded per position."""

    def __init__(self, name, wid, Hq, Hkv, D, dtype, dec_ctx, pf_prefix, pf_chunk, slack=8):
        self.dec_ctx = [int(c) for c in dec_ctx]
        self.pf_prefix = [int(p) for p in pf_prefix]
        self.pf_chunk = [int(c) for c in pf_chunk]
        self.n_dec, self.n_pf = len(self.dec_ctx), len(self.pf_prefix)
        self.ctx = np.array(self.dec_ctx + [p + c for p, c in zip(self.pf_prefix, self.pf_chunk)])
        self.w = W.small_workload(name, wid, B=len(self.ctx), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                                  sigma=0.5)
        self.nb = int(sum(W.blocks_for(int(c)) for c in self.ctx)) + slack
        self.bt = W.block_tables(self.w, self.ctx, self.nb)
        self.vals = [W.sequence_values(self.w, b, int(n), int(n)) for b, n in enumerate(self.ctx)]

    def cached_len(self, b):
        return self.dec_ctx[b] - 1 if b < self.n_dec else self.pf_prefix[b - self.n_dec]

    def fill(self, kvc):
        """A NaN pool holding every sequence's already-cached positions."""
        w, dev = self.w, "cuda"
        cache = kvc.PagedKVCache.allocate(self.nb, w.Hkv, w.D, TDTYPE[w.dtype], fill_bits=FILL)
        btd = torch.from_numpy(self.bt).to(dev)
        rows = [b for b in range(len(self.ctx)) if self.cached_len(b) > 0]
        if rows:
            seq = np.concatenate([np.full(self.cached_len(b), b, np.int32) for b in rows])
            pos = np.concatenate([np.arange(self.cached_len(b), dtype=np.int32) for b in rows])
            s = kvc.slot_mapping(btd, self.nb, torch.from_numpy(seq).to(dev),
                                 torch.from_numpy(pos).to(dev), err_flag=cache.err_flag)
            kk = np.concatenate([self.vals[b][0][:self.cached_len(b)] for b in rows])
            vv = np.concatenate([self.vals[b][1][:self.cached_len(b)] for b in rows])
            kvc.kv_append(cache, s, to_device(kk, w.dtype), to_device(vv, w.dtype))
        return cache

    def inputs(self):
        w, dev = self.w, "cuda"
        btd = torch.from_numpy(self.bt).to(dev)
        d = {}
        if self.n_dec:
            nd = self.n_dec
            d.update(
                q_decode=to_device(np.stack([self.vals[b][2][self.dec_ctx[b] - 1] for b in range(nd)]),
                                   w.dtype),
                k_new=to_device(np.stack([self.vals[b][0][self.dec_ctx[b] - 1] for b in range(nd)]),
                                w.dtype),
                v_new=to_device(np.stack([self.vals[b][1][self.dec_ctx[b] - 1] for b in range(nd)]),
                                w.dtype),
                decode_block_table=btd[:nd].contiguous(),
                decode_context_lens=torch.tensor(self.dec_ctx, dtype=torch.int32, device=dev),
                decode_max_context=max(self.dec_ctx))
        if self.n_pf:
            spans = [(self.n_dec + i, p, p + c) for i, (p, c) in
                     enumerate(zip(self.pf_prefix, self.pf_chunk))]
            cu = np.concatenate([[0], np.cumsum(self.pf_chunk)]).astype(np.int32)
            d.update(
                q_prefill=to_device(np.concatenate([self.vals[b][2][s:e] for b, s, e in spans]),
                                    w.dtype),
                k_prefill=to_device(np.concatenate([self.vals[b][0][s:e] for b, s, e in spans]),
                                    w.dtype),
                v_prefill=to_device(np.concatenate([self.vals[b][1][s:e] for b, s, e in spans]),
                                    w.dtype),
                cu_chunk_lens=torch.from_numpy(cu).to(dev),
                prefix_lens=torch.tensor(self.pf_prefix, dtype=torch.int32, device=dev),
                prefill_block_table=btd[self.n_dec:].contiguous(),
                prefill_max_chunk=max(self.pf_chunk))
        return d

    def check(self, cache, out_dec, out_pf, rows_per_chunk=None):
        w = self.w
        scale = OA.default_scale(w.D)
        worst = 0.0
        if self.n_dec:
            got = out_dec.float().cpu().numpy()
            for b in range(self.n_dec):
                k, v, q = (oracle_values(x, w.dtype) for x in self.vals[b])
                c = self.dec_ctx[b]
                ref = OA.attend_row(q[c - 1], k[:c], v[:c], scale)
                worst = max(worst, assert_close(got[b], ref, w.dtype, f"decode row {b} ctx {c}"))
        if self.n_pf:
            got = out_pf.float().cpu().numpy()
            off = 0
            for i, (p0, C) in enumerate(zip(self.pf_prefix, self.pf_chunk)):
                b = self.n_dec + i
                k, v, q = (oracle_values(x, w.dtype) for x in self.vals[b])
                rows = range(C) if rows_per_chunk is None else sorted(
                    set(np.linspace(0, C - 1, rows_per_chunk).astype(int).tolist()))
                for r in rows:
                    t = p0 + r
                    ref = OA.attend_row(q[t], k[:t + 1], v[:t + 1], scale)
                    worst = max(worst, assert_close(got[off + r], ref, w.dtype,
                                                    f"prefill chunk {i} row {r}"))
                off += C
        # every position of every sequence sits at its slot, bit for bit
        kb, vb = device_bits(cache.k_cache), device_bits(cache.v_cache)
        for b, n in enumerate(self.ctx):
            pos = np.arange(int(n))
            slots = OP.slots_for_positions(self.bt, np.full(len(pos), b), pos, 16)
            assert np.array_equal(kb[slots // 16, :, slots % 16, :],
                                  oracle_bits(self.vals[b][0], w.dtype)), f"K of sequence {b}"
            assert np.array_equal(vb[slots // 16, :, slots % 16, :],
                                  oracle_bits(self.vals[b][1], w.dtype)), f"V of sequence {b}"
        assert int(cache.err_flag.item()) == 0
        return worst


def _run(kvc, case, ws=None):
    cache = case.fill(kvc)
    out_dec, out_pf = kvc.mixed_step_attention(cache, case.w.Hq, workspace=ws, **case.inputs())
    torch.cuda.synchronize()
    return cache, out_dec, out_pf


CASES = {
    # decode contexts span 1..3 partitions of 2,048 tokens; chunks are ragged
    "bf16-32/8/128": dict(Hq=32, Hkv=8, D=128, dtype="bf16",
                          dec_ctx=[1, 2, 17, 300, 2048, 2049, 4500, 700],
                          pf_prefix=[0, 37, 300, 2000], pf_chunk=[1, 17, 300, 200]),
    "bf16-8/4/64": dict(Hq=8, Hkv=4, D=64, dtype="bf16", dec_ctx=[5, 2100, 64, 129],
                        pf_prefix=[16, 0], pf_chunk=[256, 65]),
    "fp32-4/4/32": dict(Hq=4, Hkv=4, D=32, dtype="fp32", dec_ctx=[3, 2500, 33],
                        pf_prefix=[5, 100], pf_chunk=[70, 9]),
    "fp32-16/4/32": dict(Hq=16, Hkv=4, D=32, dtype="fp32", dec_ctx=[4097, 1, 15],
                         pf_prefix=[0], pf_chunk=[130]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mixed_step_matches_oracle(kvc, name):
    cfg = CASES[name]
    say(f"mixed step {name}: decode ctx {cfg['dec_ctx']}, chunks "
        f"{list(zip(cfg['pf_prefix'], cfg['pf_chunk']))}")
    case = MixedCase(name, 400 + list(CASES).index(name), **cfg)
    cache, out_dec, out_pf = _run(kvc, case)
    worst = case.check(cache, out_dec, out_pf)
    say(f"  max abs err {worst:.2e}")


def test_mixed_prefill_rows_equal_the_prefill_kernel(kvc):
    cfg = CASES["bf16-32/8/128"]
    case = MixedCase("mixed-vs-prefill", 410, **cfg)
    say("mixed step vs chunked prefill + fused decode, bf16 32/8/128")
    cache, out_dec, out_pf = _run(kvc, case)
    ref_cache = case.fill(kvc)
    d = case.inputs()
    ref_pf = kvc.chunked_prefill_attention(ref_cache, d["q_prefill"], d["k_prefill"],
                                           d["v_prefill"], d["cu_chunk_lens"], d["prefix_lens"],
                                           d["prefill_block_table"], d["prefill_max_chunk"])
    ref_dec = kvc.decode_append_attention(ref_cache, d["q_decode"], d["k_new"], d["v_new"],
                                          d["decode_block_table"], d["decode_context_lens"],
                                          d["decode_max_context"])
    torch.cuda.synchronize()
    assert torch.equal(out_pf.view(torch.int16), ref_pf.view(torch.int16))
    assert torch.equal(cache.k_cache.view(torch.int16), ref_cache.k_cache.view(torch.int16))
    assert torch.equal(cache.v_cache.view(torch.int16), ref_cache.v_cache.view(torch.int16))
    # decode rows: another split of the same sums (8 waves per partition, not 4)
    diff = (out_dec.float() - ref_dec.float()).abs().max().item()
    assert diff <= 1e-2, diff


def test_workspace_is_reused_and_left_clean(kvc):
    """Three calls on one workspace: a small step, a larger one (more decode
    rows, so the merge counters move into what held partials), then decode
    only and prefill only; the 256-byte header is zero after each."""
    small = MixedCase("mixed-reuse-a", 420, 16, 4, 64, "bf16", [40, 3000], [10], [50])
    big = MixedCase("mixed-reuse-b", 421, 16, 4, 64, "bf16",
                    [2100 + 37 * i for i in range(40)], [0, 500], [300, 129])
    dec_only = MixedCase("mixed-reuse-c", 422, 16, 4, 64, "bf16", [5000, 7, 4200], [], [])
    pf_only = MixedCase("mixed-reuse-d", 423, 16, 4, 64, "bf16", [], [4000, 0, 3], [100, 2, 64])
    need = max(kvc.mixed_workspace_bytes(c.n_dec, max(c.dec_ctx, default=0), 16, 4, 64)
               for c in (small, big, dec_only, pf_only))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for case in (small, big, dec_only, pf_only, small):
        say(f"workspace reuse: {case.n_dec} decode rows, {case.n_pf} chunks")
        cache, out_dec, out_pf = _run(kvc, case, ws)
        case.check(cache, out_dec, out_pf)
        assert int(ws[:256].count_nonzero().item()) == 0, "queue header not reset"


def test_phase0_wait_gives_up_on_a_corrupt_header(kvc):
    """The wait for the first phase is bounded: with the workspace header's
    finished-items counter set so that it can never reach the phase-0 item
    count (a corrupt header, forced from the host), every waiting workgroup
    gives up after its spin limit, the call flags KVC_DEVERR_QUEUE and every
    workgroup still exits; the last one out leaves the header zero, and the
    next call on the same workspace is right again."""
    case = MixedCase("mixed-giveup", 424, 16, 4, 64, "bf16", [40, 300], [10, 0], [50, 70])
    need = kvc.mixed_workspace_bytes(case.n_dec, max(case.dec_ctx), 16, 4, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    hdr = ws[:12].view(torch.int32)                    # next item, phase-0 items done, exited
    hdr[1] = -1000
    say("mixed step with a corrupt queue header: the phase-0 wait must give up")
    cache = case.fill(kvc)
    kvc.mixed_step_attention(cache, case.w.Hq, workspace=ws, **case.inputs())
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & kvc.DEVERR_QUEUE
    assert int(ws[:256].count_nonzero().item()) == 0, "queue header not reset"
    cache.err_flag.zero_()
    out_dec, out_pf = kvc.mixed_step_attention(cache, case.w.Hq, workspace=ws, **case.inputs())
    torch.cuda.synchronize()
    case.check(cache, out_dec, out_pf)


def test_c4_skewed_step_in_one_launch(kvc):
    """The skewed continuous-batching step at full size (206 decode rows with
    lognormal contexts up to 32,000, 4 rows with a 2,048-token chunk), in the
    launch configuration the bench times; sampled rows against the oracle."""
    w = W.C4
    ctx = W.context_lengths(w)
    pre_rows = W.c4_prefill_rows(ctx)
    dec_rows = np.array([b for b in range(w.B) if b not in set(pre_rows.tolist())])
    chunk = W.C4_CHUNK
    rng = np.random.default_rng([w.wid, 778])
    longest = int(dec_rows[np.argmax(ctx[dec_rows])])
    sampled = sorted(set([longest] + rng.choice(dec_rows, 8, replace=False).tolist()))
    exact = sorted(set(sampled) | set(pre_rows.tolist()))
    need = int(sum(W.blocks_for(c) for c in ctx))
    nb = need + need // 100
    bt = W.block_tables(w, ctx, nb)
    say(f"C4 in one launch: {len(dec_rows)} decode rows, prefill rows {pre_rows.tolist()}")
    dev = "cuda"
    cache = kvc.PagedKVCache.allocate(nb, w.Hkv, w.D, torch.bfloat16, fill_bits=FILL)
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    cache.k_cache.normal_(0.0, w.sigma, generator=g)
    cache.v_cache.normal_(0.0, w.sigma, generator=g)
    btd = torch.from_numpy(bt).to(dev)
    vals = {}
    pre_set = set(pre_rows.tolist())
    for b in exact:
        n = int(ctx[b])
        vals[b] = W.sequence_values(w, b, n, chunk if b in pre_set else 1)
        cached = n - chunk if b in pre_set else n - 1
        if cached > 0:
            s = kvc.slot_mapping(btd, nb, torch.full((cached,), b, dtype=torch.int32, device=dev),
                                 torch.arange(cached, dtype=torch.int32, device=dev),
                                 err_flag=cache.err_flag)
            kvc.kv_append(cache, s, to_device(vals[b][0][:cached], "bf16"),
                          to_device(vals[b][1][:cached], "bf16"))
    nd = len(dec_rows)
    q_dec = torch.empty(nd, w.Hq, w.D, dtype=torch.bfloat16, device=dev).normal_(0, w.sigma, generator=g)
    k_dec = torch.empty(nd, w.Hkv, w.D, dtype=torch.bfloat16, device=dev).normal_(0, w.sigma, generator=g)
    v_dec = torch.empty_like(k_dec).normal_(0, w.sigma, generator=g)
    for i, b in enumerate(dec_rows):
        if b in vals:
            k, v, q = vals[b]
            q_dec[i], k_dec[i], v_dec[i] = (to_device(q[0], "bf16"), to_device(k[-1], "bf16"),
                                            to_device(v[-1], "bf16"))
    dsub = torch.from_numpy(dec_rows.astype(np.int64)).to(dev)
    psub = torch.from_numpy(pre_rows.astype(np.int64)).to(dev)
    out_dec, out_pf = kvc.mixed_step_attention(
        cache, w.Hq, q_decode=q_dec, k_new=k_dec, v_new=v_dec,
        decode_block_table=btd.index_select(0, dsub).contiguous(),
        decode_context_lens=torch.from_numpy(ctx[dec_rows].astype(np.int32)).to(dev),
        decode_max_context=int(ctx[dec_rows].max()),
        q_prefill=torch.cat([to_device(vals[b][2], "bf16") for b in pre_rows]),
        k_prefill=torch.cat([to_device(vals[b][0][-chunk:], "bf16") for b in pre_rows]),
        v_prefill=torch.cat([to_device(vals[b][1][-chunk:], "bf16") for b in pre_rows]),
        cu_chunk_lens=torch.arange(0, (len(pre_rows) + 1) * chunk, chunk, dtype=torch.int32,
                                   device=dev),
        prefix_lens=torch.from_numpy((ctx[pre_rows] - chunk).astype(np.int32)).to(dev),
        prefill_block_table=btd.index_select(0, psub).contiguous(), prefill_max_chunk=chunk)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    assert torch.isfinite(out_dec.float()).all() and torch.isfinite(out_pf.float()).all()
    scale = OA.default_scale(w.D)
    got = out_dec.float().cpu().numpy()
    for b in sampled:
        i = int(np.flatnonzero(dec_rows == b)[0])
        k, v, q = vals[b]
        ref = OA.attend_row(oracle_values(q[0], "bf16"), oracle_values(k, "bf16"),
                            oracle_values(v, "bf16"), scale)
        assert_close(got[i], ref, "bf16", f"C4 decode row {b} (ctx {ctx[b]})")
    got = out_pf.float().cpu().numpy()
    for i, b in enumerate(pre_rows):
        k, v, q = vals[b]
        p0 = int(ctx[b]) - chunk
        rows = [0, 1, 63, 64, 1000, chunk - 1]
        ref = np.stack([OA.attend_row(oracle_values(q[r], "bf16"),
                                      oracle_values(k[:p0 + r + 1], "bf16"),
                                      oracle_values(v[:p0 + r + 1], "bf16"), scale) for r in rows])
        assert_close(got[i * chunk + np.array(rows)], ref, "bf16", f"C4 prefill row {b}")
    # every row and head of the whole chunk of the shortest prefill row (matrix-form oracle)
    i = int(np.argmin(ctx[pre_rows]))
    b = int(pre_rows[i])
    k, v, q = vals[b]
    p0 = int(ctx[b]) - chunk
    say(f"C4 prefill row {b}: all {chunk} rows over a {p0}-token prefix")
    ref = OA.attend_positions(oracle_values(q, "bf16"), oracle_values(k, "bf16"),
                              oracle_values(v, "bf16"), p0 + np.arange(chunk), scale)
    assert_close(got[i * chunk:(i + 1) * chunk], ref, "bf16", f"C4 prefill row {b}, whole chunk")
    kb = device_bits(cache.k_cache)
    for b in exact:
        k = vals[b][0]
        n = int(ctx[b])
        for p in sorted({n - 1, n - 2, max(n - chunk, 0)}):
            s = OP.slot_of(bt[b], p, 16)
            assert np.array_equal(kb[s // 16, :, s % 16, :], oracle_bits(k[p], "bf16")), (b, p)
