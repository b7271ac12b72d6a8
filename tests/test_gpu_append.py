"""GPU parity: slot mapping and KV append are bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as OP
from tests.gpu_cases import FILL, TDTYPE, device_bits, oracle_bits, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def test_slot_mapping_bitwise(kvc):
    say("slot_mapping bitwise: 37 sequences, positions incl. padding and block edges")
    rng = np.random.default_rng(21)
    n_seqs, max_blocks, nb = 37, 9, 400
    bt = rng.permutation(nb)[:n_seqs * max_blocks].reshape(n_seqs, max_blocks).astype(np.int32)
    seq = rng.integers(0, n_seqs, 1000).astype(np.int32)
    pos = rng.integers(-3, max_blocks * 16, 1000).astype(np.int32)
    pos[:6] = [0, 15, 16, 17, 143, -1]
    want = OP.slots_for_positions(bt, seq, pos, 16)
    d = lambda a: torch.from_numpy(a).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = kvc.slot_mapping(d(bt), nb, d(seq), d(pos), err_flag=err).cpu().numpy()
    assert np.array_equal(got, want)
    assert int(err.item()) == 0


def test_slot_mapping_flags_bad_ids(kvc):
    say("slot_mapping with an out-of-range block id and sequence id")
    bt = np.array([[3, 99], [1, 2]], np.int32)       # 99 is outside a 10-block pool
    seq = np.array([0, 0, 5, 1], np.int32)
    pos = np.array([1, 20, 0, 17], np.int32)
    d = lambda a: torch.from_numpy(a).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = kvc.slot_mapping(d(bt), 10, d(seq), d(pos), err_flag=err).cpu().numpy()
    assert got.tolist() == [49, -1, -1, 2 * 16 + 1]
    assert int(err.item()) == kvc.DEVERR_BLOCK_ID | kvc.DEVERR_CONTEXT


@pytest.mark.parametrize("dtype,hkv,d", [("fp32", 4, 16), ("fp32", 2, 128), ("bf16", 8, 128),
                                         ("bf16", 3, 32)])
def test_append_bitwise_with_sentinel(kvc, dtype, hkv, d):
    say(f"kv_append bitwise {dtype} hkv={hkv} d={d}")
    rng = np.random.default_rng(22)
    nb, T = 50, 300
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[::17] = -1                                   # padding tokens write nothing
    k = rng.standard_normal((T, hkv, d)).astype(np.float32)
    v = rng.standard_normal((T, hkv, d)).astype(np.float32)
    bits = 16 if dtype == "bf16" else 32
    ek = OP.empty_pool(nb, hkv, 16, d, bits)
    ev = ek.copy()
    OP.scatter(ek, slots, oracle_bits(k, dtype))
    OP.scatter(ev, slots, oracle_bits(v, dtype))
    cache = kvc.PagedKVCache.allocate(nb, hkv, d, TDTYPE[dtype], fill_bits=FILL)
    kt, vt = to_device(k, dtype), to_device(v, dtype)
    assert np.array_equal(device_bits(kt), oracle_bits(k, dtype))   # input prep agrees
    kvc.kv_append(cache, torch.from_numpy(slots).cuda(), kt, vt)
    torch.cuda.synchronize()
    assert np.array_equal(device_bits(cache.k_cache), ek)
    assert np.array_equal(device_bits(cache.v_cache), ev)
    assert int(cache.err_flag.item()) == 0


def test_append_out_of_range_slot_is_skipped_and_flagged(kvc):
    say("kv_append with an out-of-range slot")
    nb, hkv, d = 4, 2, 16
    cache = kvc.PagedKVCache.allocate(nb, hkv, d, torch.float32, fill_bits=FILL)
    slots = torch.tensor([5, nb * 16, 10**9], dtype=torch.int64, device="cuda")
    k = torch.ones(3, hkv, d, device="cuda")
    kvc.kv_append(cache, slots, k, k)
    torch.cuda.synchronize()
    kb = device_bits(cache.k_cache)
    assert int(cache.err_flag.item()) == kvc.DEVERR_SLOT
    assert np.all(kb[0, :, 5, :] == np.float32(1).view(np.uint32))
    kb[0, :, 5, :] = 0xFFFFFFFF
    assert np.all(kb == 0xFFFFFFFF)


def test_append_then_old_blocks_unchanged(kvc):
    """Causality: appending later tokens never changes the bits of earlier ones."""
    say("append keeps earlier tokens bitwise")
    w = W.C2
    ctx = np.full(4, 40)
    bt = W.block_tables(w, ctx, 32)
    cache = kvc.PagedKVCache.allocate(32, w.Hkv, w.D, torch.float32, fill_bits=FILL)
    rng = np.random.default_rng(23)
    btd = torch.from_numpy(bt).cuda()
    snap = None
    for step in range(40):
        k = rng.standard_normal((4, w.Hkv, w.D)).astype(np.float32)
        seq = torch.arange(4, dtype=torch.int32, device="cuda")
        pos = torch.full((4,), step, dtype=torch.int32, device="cuda")
        s = kvc.slot_mapping(btd, 32, seq, pos)
        kvc.kv_append(cache, s, to_device(k, "fp32"), to_device(k, "fp32"))
        if step == 20:
            snap = device_bits(cache.k_cache).copy()
            written = snap != 0xFFFFFFFF
    torch.cuda.synchronize()
    now = device_bits(cache.k_cache)
    assert np.array_equal(now[written], snap[written])
