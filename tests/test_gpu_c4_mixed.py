"""GPU parity on the skewed continuous-batching step: 210 sequences with
lognormal context lengths (median 6,000, tail clipped at 32,000), 4 of them
mid-prefill with a 2,048-token chunk, the rest one decode token each.

The whole cache (~6.5 GB) lives on the GPU. Sequences checked against the oracle
(every prefill row, the longest decode row and 8 seeded decode rows) get their
exact seeded values; every other sequence's blocks hold seeded random data made
on the GPU, which only has to be finite for the step to be valid.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import paged as OP
from tests.gpu_cases import TDTYPE, assert_close, device_bits, oracle_bits, oracle_values, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def test_c4_skewed_mixed_step(kvc):
    w = W.C4
    ctx = W.context_lengths(w)                      # tokens held after this step
    pre_rows = W.c4_prefill_rows(ctx)
    dec_rows = np.array([b for b in range(w.B) if b not in set(pre_rows.tolist())])
    rng = np.random.default_rng([w.wid, 777])
    longest = int(dec_rows[np.argmax(ctx[dec_rows])])
    sampled_dec = sorted(set([longest] + rng.choice(dec_rows, 8, replace=False).tolist()))
    exact = sorted(set(sampled_dec) | set(pre_rows.tolist()))
    need = int(sum(W.blocks_for(c) for c in ctx))
    nb = need + need // 100
    bt = W.block_tables(w, ctx, nb)
    say(f"C4 mixed step: {w.B} sequences, sum ctx {int(ctx.sum())}, {nb} blocks, "
        f"prefill rows {pre_rows.tolist()}, exact rows {exact}")

    dev = "cuda"
    cache = kvc.PagedKVCache.allocate(nb, w.Hkv, w.D, torch.bfloat16, fill_bits=-1)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    # seeded GPU random values everywhere, then the exact sequences on top
    cache.k_cache.normal_(0.0, w.sigma, generator=g)
    cache.v_cache.normal_(0.0, w.sigma, generator=g)
    btd = torch.from_numpy(bt).to(dev)
    chunk = W.C4_CHUNK
    vals = {}
    for b in exact:
        n = int(ctx[b])
        n_q = chunk if b in set(pre_rows.tolist()) else 1
        k, v, q = W.sequence_values(w, b, n, n_q)
        vals[b] = (k, v, q)
        cached = n - chunk if b in set(pre_rows.tolist()) else n - 1
        if cached > 0:
            seq = torch.full((cached,), b, dtype=torch.int32, device=dev)
            pos = torch.arange(cached, dtype=torch.int32, device=dev)
            s = kvc.slot_mapping(btd, nb, seq, pos, err_flag=cache.err_flag)
            kvc.kv_append(cache, s, to_device(k[:cached], "bf16"), to_device(v[:cached], "bf16"))

    # decode rows: one fused append + attend launch for all 206 of them
    dsub = torch.from_numpy(dec_rows.astype(np.int64)).to(dev)
    q_dec = torch.empty(len(dec_rows), w.Hq, w.D, dtype=torch.bfloat16, device=dev).normal_(
        0.0, w.sigma, generator=g)
    k_dec = torch.empty(len(dec_rows), w.Hkv, w.D, dtype=torch.bfloat16, device=dev).normal_(
        0.0, w.sigma, generator=g)
    v_dec = torch.empty_like(k_dec).normal_(0.0, w.sigma, generator=g)
    for i, b in enumerate(dec_rows):
        if b in vals:
            k, v, q = vals[b]
            q_dec[i] = to_device(q[0], "bf16")
            k_dec[i] = to_device(k[-1], "bf16")
            v_dec[i] = to_device(v[-1], "bf16")
    bt_dec = btd.index_select(0, dsub).contiguous()
    ctx_dec = torch.from_numpy(ctx[dec_rows].astype(np.int32)).to(dev)
    out_dec = kvc.decode_append_attention(cache, q_dec, k_dec, v_dec, bt_dec, ctx_dec,
                                          int(ctx[dec_rows].max()))

    # prefill rows: one chunked-prefill launch for the 4 of them
    q_pre = torch.cat([to_device(vals[b][2], "bf16") for b in pre_rows])
    k_pre = torch.cat([to_device(vals[b][0][-chunk:], "bf16") for b in pre_rows])
    v_pre = torch.cat([to_device(vals[b][1][-chunk:], "bf16") for b in pre_rows])
    cu = torch.arange(0, (len(pre_rows) + 1) * chunk, chunk, dtype=torch.int32, device=dev)
    prefix = torch.from_numpy((ctx[pre_rows] - chunk).astype(np.int32)).to(dev)
    bt_pre = btd.index_select(0, torch.from_numpy(pre_rows.astype(np.int64)).to(dev)).contiguous()
    out_pre = kvc.chunked_prefill_attention(cache, q_pre, k_pre, v_pre, cu, prefix, bt_pre, chunk)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    assert torch.isfinite(out_dec.float()).all()

    scale = OA.default_scale(w.D)
    got_dec = out_dec.float().cpu().numpy()
    for b in sampled_dec:
        i = int(np.flatnonzero(dec_rows == b)[0])
        k, v, q = vals[b]
        ref = OA.attend_row(oracle_values(q[0], "bf16"), oracle_values(k, "bf16"),
                            oracle_values(v, "bf16"), scale)
        assert_close(got_dec[i], ref, "bf16", f"C4 decode row {b} (ctx {ctx[b]})")
    got_pre = out_pre.float().cpu().numpy()
    for i, b in enumerate(pre_rows):
        k, v, q = vals[b]
        p0 = int(ctx[b]) - chunk
        rows = [0, 1, 15, 16, 1000, chunk - 1]
        ref = np.stack([OA.attend_row(oracle_values(q[r], "bf16"), oracle_values(k[:p0 + r + 1], "bf16"),
                                      oracle_values(v[:p0 + r + 1], "bf16"), scale) for r in rows])
        assert_close(got_pre[i * chunk + np.array(rows)], ref, "bf16", f"C4 prefill row {b}")
    # every row and head of the whole chunk of the shortest prefill row (matrix-form oracle)
    i = int(np.argmin(ctx[pre_rows]))
    b = int(pre_rows[i])
    k, v, q = vals[b]
    p0 = int(ctx[b]) - chunk
    say(f"C4 prefill row {b}: all {chunk} rows over a {p0}-token prefix")
    ref = OA.attend_positions(oracle_values(q, "bf16"), oracle_values(k, "bf16"),
                              oracle_values(v, "bf16"), p0 + np.arange(chunk), scale)
    assert_close(got_pre[i * chunk:(i + 1) * chunk], ref, "bf16", f"C4 prefill row {b}, whole chunk")
    # the appended tokens and the prefill chunks landed at their slots (bitwise)
    kb = device_bits(cache.k_cache)
    for b in exact:
        k = vals[b][0]
        n = int(ctx[b])
        for p in sorted({n - 1, n - 2, max(n - chunk, 0)}):
            s = OP.slot_of(bt[b], p, 16)
            assert np.array_equal(kb[s // 16, :, s % 16, :], oracle_bits(k[p], "bf16")), (b, p)
