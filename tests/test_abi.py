"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/*.h declare, its host-only functions give the pages' numbers, and bad
arguments are rejected before any launch (no call here reaches a kernel)."""
import ctypes
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

kvc = pytest.importorskip("kv_cache_decode_append_amd")
LIB = kvc.LIB


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"kvc_kv_append", "kvc_paged_decode_attention", "kvc_chunked_prefill_attention",
            "kvc_slot_mapping", "kvc_prefix_cache_match", "kvc_prefix_cache_commit"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", kvc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvc_[a-z0-9_]+)", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert hasattr(LIB, n)


def test_kv_bytes_per_token_matches_pages():
    with open(os.path.join(ROOT, "tests", "golden", "page_numbers.json")) as f:
        page = json.load(f)
    e = page["kv_bytes_per_token"]
    assert kvc.kv_bytes_per_token(**e["args"]) == e["value"]
    e = page["kv_heads_32_kib_per_token"]
    assert kvc.kv_bytes_per_token(**e["args"]) == e["value"] * 1024
    assert kvc.kv_bytes_per_token(-1, 8, 128, 2) == -1


def test_workspace_size_closed_form():
    # one partition (<= 16 blocks) needs none
    assert kvc.decode_workspace_bytes(64, 32, 128, 256) == 0
    # 32,000 tokens = 2,000 blocks -> at most 125 partitions of >= 16 blocks
    assert kvc.decode_workspace_bytes(8, 32, 128, 32000) == 8 * 32 * 125 * (128 * 4 + 8)
    assert kvc.decode_workspace_bytes(0, 32, 128, 32000) == 0


def _cache(**over):
    c = kvc._lib._CCache(1, 1, 8, 16, 4, 16, kvc.KVC_F32, None)
    for k, v in over.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("over,status", [
    (dict(k_cache=None), -1),
    (dict(dtype=7), -3),
    (dict(block_size=32), -4),
    (dict(head_dim=48), -4),
    (dict(num_kv_heads=0), -2),
])
def test_bad_cache_rejected_before_launch(over, status):
    c = _cache(**over)
    assert LIB.kvc_kv_append(ctypes.byref(c), 1, 1, 1, 4, None) == status
    assert LIB.kvc_paged_decode_attention(ctypes.byref(c), 1, 1, 4, 1, 4, 1, 64, 0.25, 1,
                                          None, 0, None) == status


def test_bad_shapes_rejected_before_launch():
    c = _cache()
    byref = ctypes.byref(c)
    # Hq not a multiple of Hkv
    assert LIB.kvc_paged_decode_attention(byref, 1, 1, 6, 1, 4, 1, 64, 0.25, 1, None, 0, None) == -2
    # G = 3 is not supported
    assert LIB.kvc_paged_decode_attention(byref, 1, 1, 12, 1, 4, 1, 64, 0.25, 1, None, 0, None) == -4
    # context longer than the block table
    assert LIB.kvc_paged_decode_attention(byref, 1, 1, 4, 1, 4, 1, 65, 0.25, 1, None, 0, None) == -2
    # split-K needed but no workspace
    assert LIB.kvc_paged_decode_attention(byref, 1, 1, 4, 1, 400, 1, 6400, 0.25, 1, None, 0,
                                          None) == -5
    # null q
    assert LIB.kvc_paged_decode_attention(byref, None, 1, 4, 1, 4, 1, 64, 0.25, 1, None, 0,
                                          None) == -1
    assert LIB.kvc_kv_append(byref, 1, 1, 1, -1, None) == -2
    assert LIB.kvc_kv_append(byref, None, 1, 1, 3, None) == -1
    assert LIB.kvc_slot_mapping(1, 1, 4, 8, 1, 1, 5, 8, 1, None, None) == -4
    assert LIB.kvc_slot_mapping(None, 1, 4, 8, 1, 1, 5, 16, 1, None, None) == -1
    assert LIB.kvc_slot_mapping(1, 1, 4, 8, 1, 1, -5, 16, 1, None, None) == -2


def test_prefill_split_workspace_rules():
    # 208 query tokens over a 2,000-token context, GQA 32/8/128: 8 key-range splits
    assert kvc.prefill_workspace_bytes(1, 208, 208, 2000, 32, 8, 128) == 208 * 32 * 8 * (128 * 4 + 8)
    # enough query tiles already (8 x 2,048 tokens): no split, no workspace
    assert kvc.prefill_workspace_bytes(8, 16384, 2048, 32048, 32, 8, 128) == 0
    assert kvc.prefill_workspace_bytes(1, 208, 208, 100, 32, 8, 128) == 0   # context < chunk
    c = _cache(num_kv_heads=2, head_dim=64)
    byref = ctypes.byref(c)
    args = (byref, 1, 1, 1, 1, 1, 1, 208, 208)
    tail = (1, 200, 8, 0.125, 1)
    # split needed, workspace missing or one byte short
    need = kvc.prefill_workspace_bytes(1, 208, 208, 2000, 8, 2, 64)
    assert need > 0
    assert LIB.kvc_chunked_prefill_attention_split(*args, 2000, *tail, None, 0, None) == -5
    assert LIB.kvc_chunked_prefill_attention_split(*args, 2000, *tail, 1, need - 1, None) == -5
    # the context bound below the chunk, or negative
    assert LIB.kvc_chunked_prefill_attention_split(*args, 100, *tail, 1, need, None) == -2
    assert LIB.kvc_chunked_prefill_attention_split(*args, -1, *tail, 1, need, None) == -2


def test_zero_sized_calls_launch_nothing():
    c = _cache()
    assert LIB.kvc_kv_append(ctypes.byref(c), 1, 1, 1, 0, None) == 0
    assert LIB.kvc_paged_decode_attention(ctypes.byref(c), 1, 0, 4, 1, 4, 1, 64, 0.25, 1, None,
                                          0, None) == 0
    assert LIB.kvc_slot_mapping(1, 1, 4, 8, 1, 1, 0, 16, 1, None, None) == 0


def test_status_strings():
    for s in range(-10, 1):
        assert LIB.kvc_status_string(s)
    assert LIB.kvc_status_string(-99) == b"unknown status"


def _mixed(**over):
    b = kvc._lib._CMixed()
    for k, v in over.items():
        setattr(b, k, v)
    return b


def test_mixed_workspace_closed_form():
    # the queue header, then one int per decode row (rounded up to 256 bytes)
    assert kvc.mixed_workspace_bytes(0, 0, 32, 8, 128) == 256
    assert kvc.mixed_workspace_bytes(64, 2048, 32, 8, 128) == 512
    assert kvc.mixed_workspace_bytes(206, 32000, 32, 8, 128) == 256 + 1024
    assert kvc.mixed_workspace_bytes(4096, 32000, 32, 8, 128) == 256 + 16384
    assert kvc.mixed_workspace_bytes(4097, 16, 32, 8, 128) == 0
    assert kvc.mixed_workspace_bytes(4, 16, 6, 4, 128) == 0


def test_mixed_step_rejects_before_launch():
    c = _cache(num_kv_heads=2, head_dim=32)
    byref = ctypes.byref(c)
    ws = kvc.mixed_workspace_bytes(2, 100, 4, 2, 32)
    dec = dict(n_decode=2, q_decode=1, k_new=1, v_new=1, decode_block_table=1,
               decode_max_blocks=8, decode_context_lens=1, decode_max_context=100, out_decode=1)
    f = LIB.kvc_mixed_step_attention
    assert f(byref, None, 4, 0.1, 1, ws, None) == -1                       # no batch
    assert f(byref, ctypes.byref(_mixed()), 4, 0.1, None, 0, None) == 0    # nothing to do
    assert f(byref, ctypes.byref(_mixed(**dec)), 4, 0.1, None, 0, None) == -5   # no workspace
    assert f(byref, ctypes.byref(_mixed(**dec)), 4, 0.1, 1, ws - 1, None) == -5
    assert f(byref, ctypes.byref(_mixed(**dict(dec, q_decode=None))), 4, 0.1, 1, ws, None) == -1
    assert f(byref, ctypes.byref(_mixed(**dict(dec, decode_max_context=129))), 4, 0.1, 1, ws,
             None) == -2                                                    # beyond 8 blocks
    assert f(byref, ctypes.byref(_mixed(**dict(dec, n_decode=4097))), 4, 0.1, 1, 1 << 30,
             None) == -4
    assert f(byref, ctypes.byref(_mixed(**dec)), 16, 0.1, 1, 1 << 30, None) == -4   # G = 8
    assert f(byref, ctypes.byref(_mixed(**dec)), 6, 0.1, 1, 1 << 30, None) == -4   # G = 3
    assert f(byref, ctypes.byref(_mixed(**dec)), 5, 0.1, 1, 1 << 30, None) == -2   # 5 % 2 != 0
    c64 = _cache(num_kv_heads=2, head_dim=64)
    assert f(ctypes.byref(c64), ctypes.byref(_mixed(**dec)), 4, 0.1, 1, 1 << 30, None) == -4
    pf = dict(n_prefill=1, q_prefill=1, k_prefill=1, v_prefill=1, cu_chunk_lens=1, prefix_lens=1,
              prefill_total_tokens=10, prefill_max_chunk=10, prefill_block_table=1,
              prefill_max_blocks=4, out_prefill=None)
    assert f(byref, ctypes.byref(_mixed(**pf)), 4, 0.1, 1, 1 << 30, None) == -1


def test_fp8_cache_rules():
    c = _cache(dtype=2, head_dim=64)                  # no scale pools
    byref = ctypes.byref(c)
    assert LIB.kvc_kv_append(byref, 1, 1, 1, 4, None) == -1
    c = _cache(dtype=2, head_dim=32, k_scale=1, v_scale=1)
    assert LIB.kvc_kv_append(ctypes.byref(c), 1, 1, 1, 4, None) == -4
    c = _cache(dtype=2, head_dim=64, k_scale=1, v_scale=1)
    byref = ctypes.byref(c)
    assert LIB.kvc_kv_append(byref, 1, 1, 1, 0, None) == 0
    # the mixed step takes an fp8 cache of head_dim 64 or 128 (here: nothing to do)
    assert LIB.kvc_mixed_step_attention(byref, ctypes.byref(_mixed()), 4, 0.1, 1, 256, None) == 0
    c32 = _cache(dtype=2, head_dim=32, k_scale=1, v_scale=1)
    assert LIB.kvc_mixed_step_attention(ctypes.byref(c32), ctypes.byref(_mixed()), 4, 0.1, 1, 256,
                                        None) == -4
    assert kvc.KVC_FP8 == 2


ALIGN = -10
A = 1 << 12                # an aligned placeholder address (never dereferenced: every call
                           # below is rejected on the host before any launch)


def test_misaligned_pointers_rejected_before_launch():
    """Each call is valid but for one pointer's alignment (16 bytes for tensors
    and pools, 4 for int32 arrays, 8 for slot lists), so KVC_ERR_ALIGN is what
    stops it."""
    assert kvc._lib.LIB.kvc_status_string(ALIGN) != b"unknown status"
    c = _cache(k_cache=A, v_cache=A)
    byref = ctypes.byref(c)
    # append: k, the slot list, the pool
    assert LIB.kvc_kv_append(byref, A, A + 2, A, 4, None) == ALIGN
    assert LIB.kvc_kv_append(byref, A + 4, A, A, 4, None) == ALIGN
    c_bad = _cache(k_cache=A + 8, v_cache=A)
    assert LIB.kvc_kv_append(ctypes.byref(c_bad), A, A, A, 4, None) == ALIGN
    # slot mapping: the int64 output, an int32 input
    assert LIB.kvc_slot_mapping(A, 1, 4, 8, A, A, 5, 16, A + 4, None, None) == ALIGN
    assert LIB.kvc_slot_mapping(A, 1, 4, 8, A + 2, A, 5, 16, A, None, None) == ALIGN
    # decode: q, out, the block table
    dec = [A, 1, 4, A, 4, A, 64, 0.25, A, None, 0, None]
    for i, bad in ((0, A + 4), (8, A + 8), (3, A + 2)):
        args = list(dec)
        args[i] = bad
        assert LIB.kvc_paged_decode_attention(byref, *args) == ALIGN, i
    # fused decode: k_new
    assert LIB.kvc_decode_append_attention(byref, A, A + 4, A, 1, 4, A, 4, A, 64, 0.25, A, None,
                                           0, None) == ALIGN
    # chunked prefill: q, then cu_chunk_lens
    pf = [A, A, A, 1, A, A, 8, 8, A, 4, 4, 0.25, A, None]
    for i, bad in ((0, A + 6), (4, A + 1)):
        args = list(pf)
        args[i] = bad
        assert LIB.kvc_chunked_prefill_attention(byref, *args) == ALIGN, i
    # mixed step: a decode row's query, and the workspace
    c32 = _cache(k_cache=A, v_cache=A, num_kv_heads=2, head_dim=32)
    dec_rows = dict(n_decode=2, q_decode=A + 4, k_new=A, v_new=A, decode_block_table=A,
                    decode_max_blocks=8, decode_context_lens=A, decode_max_context=100,
                    out_decode=A)
    ws = kvc.mixed_workspace_bytes(2, 100, 4, 2, 32)
    f = LIB.kvc_mixed_step_attention
    assert f(ctypes.byref(c32), ctypes.byref(_mixed(**dec_rows)), 4, 0.1, A, ws, None) == ALIGN
    assert f(ctypes.byref(c32), ctypes.byref(_mixed(**dict(dec_rows, q_decode=A))), 4, 0.1, A + 8,
             ws, None) == ALIGN
    # the read probe: data, then a size that is not a multiple of 16
    assert LIB.kvc_stream_read(A + 4, 16, A, None) == ALIGN
    assert LIB.kvc_stream_read(A, 8, A, None) == -2
