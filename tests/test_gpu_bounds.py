"""GPU: decode rows whose context length exceeds the host-given bound.

The fused append + decode launch and the one-launch mixed step read each
row's context length from device memory and size their work by a host-known
bound (max_context_len). A row past that bound is a caller error. The kernels
flag it with KVC_DEVERR_CONTEXT, attend the row over the first bound tokens,
and append nothing for it: the new token's position lies past the bound, and
the clamped position holds a valid cached token that must not be overwritten.
The other rows of the call are appended and attended as usual.

Each test snapshots the pool after the cached tokens are written, makes the
call, and checks that exactly the in-bound rows' new-token slots changed, to
the oracle's bits; the outputs are checked against the oracle's attention
(the clamped row over its first `bound` tokens).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import paged as OP
from oracle import quant as OQ
from tests.gpu_cases import (FILL, TDTYPE, assert_close, device_bits, oracle_bits, oracle_values,
                             say, to_device)

pytestmark = pytest.mark.gpu
KVC_DEVERR_CONTEXT = 4
CTX = [40, 100, 70]      # row 1 runs past the bound
BOUND = 80


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def _setup(kvc, name, wid, dtype_t):
    """Seeded values for CTX, a NaN pool holding positions 0 .. ctx - 2 of every
    row, and the device block table."""
    w = W.small_workload(name, wid, B=len(CTX), Hq=32, Hkv=8, D=128, dtype="bf16", sigma=0.5)
    ctx = np.asarray(CTX, np.int64)
    nb = int(sum(W.blocks_for(int(c)) for c in ctx)) + 4
    bt = W.block_tables(w, ctx, nb)
    vals = [W.sequence_values(w, b, int(n), int(n)) for b, n in enumerate(ctx)]
    cache = kvc.PagedKVCache.allocate(nb, w.Hkv, w.D, dtype_t, fill_bits=FILL)
    btd = torch.from_numpy(bt).cuda()
    seq = np.concatenate([np.full(int(n) - 1, b, np.int32) for b, n in enumerate(ctx)])
    pos = np.concatenate([np.arange(int(n) - 1, dtype=np.int32) for n in ctx])
    s = kvc.slot_mapping(btd, nb, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                         err_flag=cache.err_flag)
    kvc.kv_append(cache, s, to_device(np.concatenate([v[0][:-1] for v in vals]), "bf16"),
                  to_device(np.concatenate([v[1][:-1] for v in vals]), "bf16"))
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    return w, ctx, nb, bt, btd, vals, cache


def _pool_bytes(cache):
    out = [cache.k_cache.view(torch.uint8).cpu().numpy().copy(),
           cache.v_cache.view(torch.uint8).cpu().numpy().copy()]
    if cache.k_scale is not None:
        out += [cache.k_scale.view(torch.uint8).cpu().numpy().copy(),
                cache.v_scale.view(torch.uint8).cpu().numpy().copy()]
    return out


def _changed_slots(before, after):
    """Slots (block * 16 + offset) where any byte of any pool differs."""
    slots = set()
    for x, y in zip(before, after):
        diff = (x != y).reshape(x.shape[0], x.shape[1], 16, -1).any(axis=(1, 3))
        blk, off = np.nonzero(diff)
        slots.update((blk * 16 + off).tolist())
    return slots


def _new_slots(bt, rows):
    return {int(OP.slots_for_positions(bt, [b], [CTX[b] - 1], 16)[0]) for b in rows}


def _check_outputs(w, vals, got, dequant=None):
    scale = OA.default_scale(w.D)
    for b, c in enumerate(CTX):
        n = min(c, BOUND)
        k, v, q = (oracle_values(x, "bf16") for x in vals[b])
        if dequant is not None:
            k, v = dequant(k), dequant(v)
        ref = OA.attend_row(q[c - 1], k[:n], v[:n], scale)
        assert_close(got[b], ref, "bf16", f"row {b} ctx {c} bound {BOUND}")


def test_fused_decode_skips_the_append_of_a_row_past_the_bound(kvc):
    say(f"fused decode bf16, ctx {CTX}, bound {BOUND}")
    w, ctx, nb, bt, btd, vals, cache = _setup(kvc, "bound-bf16", 9101, torch.bfloat16)
    before = _pool_bytes(cache)
    q = to_device(np.stack([v[2][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    kn = to_device(np.stack([v[0][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    vn = to_device(np.stack([v[1][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    lens = torch.tensor(CTX, dtype=torch.int32, device="cuda")
    out = kvc.decode_append_attention(cache, q, kn, vn, btd, lens, BOUND)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & KVC_DEVERR_CONTEXT
    after = _pool_bytes(cache)
    assert _changed_slots(before, after) == _new_slots(bt, [0, 2])
    kb, vb = device_bits(cache.k_cache), device_bits(cache.v_cache)
    for b in (0, 2):
        s = _new_slots(bt, [b]).pop()
        assert np.array_equal(kb[s // 16, :, s % 16, :], oracle_bits(vals[b][0][-1], "bf16"))
        assert np.array_equal(vb[s // 16, :, s % 16, :], oracle_bits(vals[b][1][-1], "bf16"))
    _check_outputs(w, vals, out.float().cpu().numpy())


def test_fused_fp8_decode_skips_the_append_of_a_row_past_the_bound(kvc):
    say(f"fused decode fp8, ctx {CTX}, bound {BOUND}")
    w, ctx, nb, bt, btd, vals, cache = _setup(kvc, "bound-fp8", 9102, torch.float8_e4m3fn)
    before = _pool_bytes(cache)
    q = to_device(np.stack([v[2][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    kn = to_device(np.stack([v[0][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    vn = to_device(np.stack([v[1][c - 1] for v, c in zip(vals, CTX)]), "bf16")
    lens = torch.tensor(CTX, dtype=torch.int32, device="cuda")
    out = kvc.decode_append_attention(cache, q, kn, vn, btd, lens, BOUND)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & KVC_DEVERR_CONTEXT
    after = _pool_bytes(cache)
    assert _changed_slots(before, after) == _new_slots(bt, [0, 2])
    kc = cache.k_cache.view(torch.uint8).cpu().numpy()
    ks = cache.k_scale.cpu().numpy()
    for b in (0, 2):
        s = _new_slots(bt, [b]).pop()
        codes, scales = OQ.quantize_rows(oracle_values(vals[b][0][-1:], "bf16").astype(np.float32))
        assert np.array_equal(kc[s // 16, :, s % 16, :], codes[0])
        assert np.array_equal(ks[s // 16, :, s % 16].view(np.uint32), scales[0].view(np.uint32))

    def dequant(x):
        return OQ.dequantize_rows(*OQ.quantize_rows(x.astype(np.float32)))
    _check_outputs(w, vals, out.float().cpu().numpy(), dequant)


@pytest.mark.parametrize("fp8", [False, True])
def test_mixed_step_skips_the_append_of_a_row_past_the_bound(kvc, fp8):
    say(f"mixed step {'fp8' if fp8 else 'bf16'}, decode ctx {CTX}, bound {BOUND}")
    dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    w, ctx, nb, bt, btd, vals, cache = _setup(kvc, f"bound-mixed-{int(fp8)}", 9103 + fp8, dt)
    before = _pool_bytes(cache)
    out_dec, _ = kvc.mixed_step_attention(
        cache, w.Hq,
        q_decode=to_device(np.stack([v[2][c - 1] for v, c in zip(vals, CTX)]), "bf16"),
        k_new=to_device(np.stack([v[0][c - 1] for v, c in zip(vals, CTX)]), "bf16"),
        v_new=to_device(np.stack([v[1][c - 1] for v, c in zip(vals, CTX)]), "bf16"),
        decode_block_table=btd, decode_context_lens=torch.tensor(CTX, dtype=torch.int32,
                                                                 device="cuda"),
        decode_max_context=BOUND)
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) & KVC_DEVERR_CONTEXT
    assert _changed_slots(before, _pool_bytes(cache)) == _new_slots(bt, [0, 2])
    dequant = (lambda x: OQ.dequantize_rows(*OQ.quantize_rows(x.astype(np.float32)))) if fp8 \
        else None
    _check_outputs(w, vals, out_dec.float().cpu().numpy(), dequant)
