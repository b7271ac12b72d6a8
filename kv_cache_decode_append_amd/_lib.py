"""ctypes binding for libkvc.so: argument marshalling only.

Every function here checks tensor dtypes, devices and shapes, passes raw device
pointers plus torch's current HIP stream to the C ABI declared in
include/kvc.h, and raises on a negative status. All computation happens in the
HIP kernels; there is no fallback path. If the library is missing or cannot be
loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_F32, KVC_BF16, KVC_FP8 = 0, 1, 2
DEVERR_BLOCK_ID, DEVERR_SLOT, DEVERR_CONTEXT, DEVERR_QUEUE = 1, 2, 4, 8
BLOCK_SIZE = 16

_DTYPE_CODE = {torch.float32: KVC_F32, torch.bfloat16: KVC_BF16, torch.float8_e4m3fn: KVC_FP8}


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class _CCache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("err_flag", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class _CStep(ctypes.Structure):
    """kvc_step (include/kvc_sched.h)."""
    _p = ctypes.POINTER(ctypes.c_int32)
    _fields_ = [("n_decode", ctypes.c_int32), ("decode_ids", _p), ("decode_context_lens", _p),
                ("decode_block_table", _p), ("decode_max_context", ctypes.c_int32),
                ("n_prefill", ctypes.c_int32), ("prefill_ids", _p), ("prefill_prefix_lens", _p),
                ("prefill_cu_chunk_lens", _p), ("prefill_block_table", _p),
                ("prefill_total_tokens", ctypes.c_int32), ("prefill_max_chunk", ctypes.c_int32),
                ("prefill_max_context", ctypes.c_int32),
                ("n_first", ctypes.c_int32), ("first_token_ids", _p),
                ("n_finished", ctypes.c_int32), ("finished_ids", _p)]


class _CMixed(ctypes.Structure):
    """kvc_mixed_batch (include/kvc.h)."""
    _fields_ = [("n_decode", ctypes.c_int32), ("q_decode", ctypes.c_void_p),
                ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("decode_block_table", ctypes.c_void_p), ("decode_max_blocks", ctypes.c_int32),
                ("decode_context_lens", ctypes.c_void_p), ("decode_max_context", ctypes.c_int32),
                ("out_decode", ctypes.c_void_p),
                ("n_prefill", ctypes.c_int32), ("q_prefill", ctypes.c_void_p),
                ("k_prefill", ctypes.c_void_p), ("v_prefill", ctypes.c_void_p),
                ("cu_chunk_lens", ctypes.c_void_p), ("prefix_lens", ctypes.c_void_p),
                ("prefill_total_tokens", ctypes.c_int32), ("prefill_max_chunk", ctypes.c_int32),
                ("prefill_block_table", ctypes.c_void_p), ("prefill_max_blocks", ctypes.c_int32),
                ("out_prefill", ctypes.c_void_p)]


def _hip_runtimes_mapped() -> set[str]:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python kv_cache_decode_append_amd/build.py`")
    # torch's own HIP runtime must already be mapped so that the library binds
    # to it (same soname) instead of loading a second runtime.
    import torch.cuda  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped in this process: {sorted(runtimes)}")
    c_int, c_i32, c_i64, c_sz = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    vp, fl = ctypes.c_void_p, ctypes.c_float
    P = ctypes.POINTER(_CCache)
    sig = {
        "kvc_kv_bytes_per_token": (c_i64, [c_i32, c_i32, c_i32, c_i32]),
        "kvc_slot_mapping": (c_int, [vp, c_i32, c_i32, c_i32, vp, vp, c_i32, c_i32, vp, vp, vp]),
        "kvc_kv_append": (c_int, [P, vp, vp, vp, c_i32, vp]),
        "kvc_decode_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
        "kvc_paged_decode_attention": (c_int, [P, vp, c_i32, c_i32, vp, c_i32, vp, c_i32, fl, vp,
                                               vp, c_sz, vp]),
        "kvc_decode_append_attention": (c_int, [P, vp, vp, vp, c_i32, c_i32, vp, c_i32, vp, c_i32,
                                                fl, vp, vp, c_sz, vp]),
        "kvc_decode_append_attention_noalloc": (c_int, [P, vp, vp, vp, c_i32, c_i32, vp, c_i32, vp,
                                                        c_i32, fl, vp, vp]),
        "kvc_chunked_prefill_attention": (c_int, [P, vp, vp, vp, c_i32, vp, vp, c_i32, c_i32, vp,
                                                  c_i32, c_i32, fl, vp, vp]),
        "kvc_prefill_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
        "kvc_chunked_prefill_attention_split": (c_int, [P, vp, vp, vp, c_i32, vp, vp, c_i32, c_i32,
                                                        c_i32, vp, c_i32, c_i32, fl, vp, vp, c_sz,
                                                        vp]),
        "kvc_status_string": (ctypes.c_char_p, [c_int]),
        "kvc_prefix_cache_create": (vp, [c_i32, c_i32]),
        "kvc_prefix_cache_destroy": (None, [vp]),
        "kvc_prefix_cache_match": (c_i32, [vp, vp, c_i32, vp, c_i32]),
        "kvc_prefix_cache_allocate": (c_i32, [vp, c_i32, vp]),
        "kvc_prefix_cache_commit": (c_i32, [vp, vp, c_i32, vp, c_i32]),
        "kvc_prefix_cache_release": (c_i32, [vp, vp, c_i32]),
        "kvc_prefix_cache_refcount": (c_i32, [vp, c_i32]),
        "kvc_prefix_cache_counts": (c_i32, [vp, vp, vp, vp]),
        "kvc_mixed_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
        "kvc_mixed_step_attention": (c_int, [P, ctypes.POINTER(_CMixed), c_i32, fl, vp, c_sz, vp]),
        "kvc_sched_create": (vp, [c_i32, c_i32, c_i32, c_i32, c_i32]),
        "kvc_sched_destroy": (None, [vp]),
        "kvc_sched_submit": (c_i32, [vp, c_i32, c_i32]),
        "kvc_sched_unfinished": (c_i32, [vp]),
        "kvc_sched_next_step": (c_i32, [vp, ctypes.POINTER(_CStep)]),
        "kvc_stream_read_groups": (c_i32, []),
        "kvc_stream_read": (c_int, [vp, c_sz, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvcError(fn, status, LIB.kvc_status_string(status).decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class PagedKVCache:
    """One layer's K and V block pools, [num_blocks, Hkv, 16, head_dim] each.

    The tensors are owned by the caller (allocated here with torch for
    convenience); the library only reads and writes them. A float8_e4m3fn
    cache also has K and V row scales, [num_blocks, Hkv, 16] float32 each;
    its queries, new K/V and outputs are bfloat16 (``dtype``).
    """

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 err_flag: torch.Tensor | None = None, k_scale: torch.Tensor | None = None,
                 v_scale: torch.Tensor | None = None):
        _need(k_cache, "k_cache", ndim=4)
        _need(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4, device=k_cache.device)
        if k_cache.shape != v_cache.shape:
            raise ValueError("k_cache and v_cache shapes differ")
        if k_cache.dtype not in _DTYPE_CODE:
            raise TypeError(f"cache dtype {k_cache.dtype} is not fp32, bf16 or float8_e4m3fn")
        if k_cache.shape[2] != BLOCK_SIZE:
            raise ValueError("block size must be 16")
        if err_flag is not None:
            _need(err_flag, "err_flag", dtype=torch.int32, device=k_cache.device)
        nb, hkv, _, d = k_cache.shape
        fp8 = k_cache.dtype == torch.float8_e4m3fn
        if fp8:
            for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
                _need(t, n, torch.float32, 3, k_cache.device)
                if t.shape != (nb, hkv, BLOCK_SIZE):
                    raise ValueError(f"{n} must be [{nb}, {hkv}, {BLOCK_SIZE}]")
        elif k_scale is not None or v_scale is not None:
            raise ValueError("row scales belong to a float8_e4m3fn cache only")
        self.k_cache, self.v_cache, self.err_flag = k_cache, v_cache, err_flag
        self.k_scale, self.v_scale = k_scale, v_scale
        self.num_blocks, self.num_kv_heads, self.head_dim = nb, hkv, d
        self.storage_dtype = k_cache.dtype
        self.dtype = torch.bfloat16 if fp8 else k_cache.dtype
        self._c = _CCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, BLOCK_SIZE, hkv, d,
                          _DTYPE_CODE[k_cache.dtype], _ptr(err_flag), _ptr(k_scale), _ptr(v_scale))

    @classmethod
    def allocate(cls, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device="cuda", with_err_flag: bool = True, fill_bits: int | None = None):
        shape = (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim)
        k = torch.empty(shape, dtype=dtype, device=device)
        v = torch.empty(shape, dtype=dtype, device=device)
        ks = vs = None
        if dtype == torch.float8_e4m3fn:
            ks = torch.empty(shape[:3], dtype=torch.float32, device=device)
            vs = torch.empty(shape[:3], dtype=torch.float32, device=device)
        if fill_bits is not None:
            ib = {torch.bfloat16: torch.int16, torch.float8_e4m3fn: torch.int8}.get(dtype, torch.int32)
            k.view(ib).fill_(fill_bits)
            v.view(ib).fill_(fill_bits)
            if ks is not None:
                ks.view(torch.int32).fill_(fill_bits)
                vs.view(torch.int32).fill_(fill_bits)
        err = torch.zeros(1, dtype=torch.int32, device=device) if with_err_flag else None
        return cls(k, v, err, ks, vs)

    @property
    def c(self):
        return ctypes.byref(self._c)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(LIB.kvc_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def slot_mapping(block_table: torch.Tensor, num_blocks: int, seq_ids: torch.Tensor,
                 positions: torch.Tensor, out: torch.Tensor | None = None,
                 err_flag: torch.Tensor | None = None) -> torch.Tensor:
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_ids, "seq_ids", torch.int32, 1, block_table.device)
    _need(positions, "positions", torch.int32, 1, block_table.device)
    T = positions.shape[0]
    if seq_ids.shape[0] != T:
        raise ValueError("seq_ids and positions differ in length")
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=block_table.device)
    _need(out, "slot_mapping", torch.int64, 1, block_table.device)
    if err_flag is not None:
        _need(err_flag, "err_flag", torch.int32, 1, block_table.device)
    _check("kvc_slot_mapping", LIB.kvc_slot_mapping(
        block_table.data_ptr(), block_table.shape[0], block_table.shape[1], num_blocks,
        seq_ids.data_ptr(), positions.data_ptr(), T, BLOCK_SIZE, out.data_ptr(),
        _ptr(err_flag), _stream()))
    return out


def kv_append(cache: PagedKVCache, slot_mapping: torch.Tensor, k: torch.Tensor,
              v: torch.Tensor) -> None:
    _need(slot_mapping, "slot_mapping", torch.int64, 1, cache.k_cache.device)
    _need(k, "k", cache.dtype, 3, cache.k_cache.device)
    _need(v, "v", cache.dtype, 3, cache.k_cache.device)
    T = slot_mapping.shape[0]
    if k.shape != (T, cache.num_kv_heads, cache.head_dim) or v.shape != k.shape:
        raise ValueError(f"k/v must be [{T}, {cache.num_kv_heads}, {cache.head_dim}]")
    _check("kvc_kv_append", LIB.kvc_kv_append(cache.c, slot_mapping.data_ptr(), k.data_ptr(),
                                              v.data_ptr(), T, _stream()))


def decode_workspace_bytes(B: int, Hq: int, head_dim: int, max_context_len: int) -> int:
    return int(LIB.kvc_decode_workspace_bytes(B, Hq, head_dim, max_context_len))


def _decode(cache, q, k_new, v_new, block_table, context_lens, max_context_len, softmax_scale,
            out, workspace, noalloc=False):
    dev = cache.k_cache.device
    _need(q, "q", cache.dtype, 3, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    if D != cache.head_dim or block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("q / block_table / context_lens shapes disagree")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _need(t, n, cache.dtype, 3, dev)
            if t.shape != (B, cache.num_kv_heads, D):
                raise ValueError(f"{n} must be [{B}, {cache.num_kv_heads}, {D}]")
    if out is None:
        if noalloc:
            raise ValueError("out is required (this call allocates nothing)")
        out = torch.empty_like(q)
    _need(out, "out", cache.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if noalloc:
        scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
        _check("kvc_decode_append_attention_noalloc", LIB.kvc_decode_append_attention_noalloc(
            cache.c, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), B, Hq,
            block_table.data_ptr(), block_table.shape[1], context_lens.data_ptr(),
            int(max_context_len), scale, out.data_ptr(), _stream()))
        return out
    need = decode_workspace_bytes(B, Hq, D, max_context_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None:
        _need(workspace, "workspace", device=dev)
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    if k_new is None:
        _check("kvc_paged_decode_attention", LIB.kvc_paged_decode_attention(
            cache.c, q.data_ptr(), B, Hq, block_table.data_ptr(), block_table.shape[1],
            context_lens.data_ptr(), int(max_context_len), scale, out.data_ptr(),
            _ptr(workspace), ws_bytes, _stream()))
    else:
        _check("kvc_decode_append_attention", LIB.kvc_decode_append_attention(
            cache.c, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), B, Hq,
            block_table.data_ptr(), block_table.shape[1], context_lens.data_ptr(),
            int(max_context_len), scale, out.data_ptr(), _ptr(workspace), ws_bytes, _stream()))
    return out


def paged_decode_attention(cache: PagedKVCache, q: torch.Tensor, block_table: torch.Tensor,
                           context_lens: torch.Tensor, max_context_len: int,
                           softmax_scale: float | None = None, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Attend each q[b] over positions 0 .. context_lens[b]-1 of its cached K/V."""
    return _decode(cache, q, None, None, block_table, context_lens, max_context_len,
                   softmax_scale, out, workspace)


def decode_append_attention(cache: PagedKVCache, q: torch.Tensor, k_new: torch.Tensor,
                            v_new: torch.Tensor, block_table: torch.Tensor,
                            context_lens: torch.Tensor, max_context_len: int,
                            softmax_scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One fused decode step: append k_new/v_new at position context_lens[b]-1, then attend."""
    return _decode(cache, q, k_new, v_new, block_table, context_lens, max_context_len,
                   softmax_scale, out, workspace)


def decode_append_attention_noalloc(cache: PagedKVCache, q: torch.Tensor, k_new: torch.Tensor,
                                    v_new: torch.Tensor, block_table: torch.Tensor,
                                    context_lens: torch.Tensor, max_context_len: int,
                                    out: torch.Tensor,
                                    softmax_scale: float | None = None) -> torch.Tensor:
    """decode_append_attention with no workspace and no allocation, for callers
    that cannot allocate (kvc_decode_append_attention_noalloc: the split-K
    partials use the library's per-device scratch array). ``out`` is required."""
    if k_new is None or v_new is None:
        raise ValueError("k_new and v_new are required")
    return _decode(cache, q, k_new, v_new, block_table, context_lens, max_context_len,
                   softmax_scale, out, None, noalloc=True)


def prefill_workspace_bytes(n_seqs: int, total_tokens: int, max_chunk_len: int,
                            max_context_len: int, Hq: int, num_kv_heads: int, head_dim: int) -> int:
    return int(LIB.kvc_prefill_workspace_bytes(n_seqs, total_tokens, max_chunk_len,
                                               max_context_len, Hq, num_kv_heads, head_dim))


def chunked_prefill_attention(cache: PagedKVCache, q: torch.Tensor, k: torch.Tensor,
                              v: torch.Tensor, cu_chunk_lens: torch.Tensor,
                              prefix_lens: torch.Tensor, block_table: torch.Tensor,
                              max_chunk_len: int, softmax_scale: float | None = None,
                              out: torch.Tensor | None = None, max_context_len: int | None = None,
                              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """With ``max_context_len`` (a bound on prefix + chunk) the call may split
    each query tile's keys over several workgroups (kvc_chunked_prefill_attention_split);
    a workspace of the size the library asks for is allocated here when none
    is given."""
    dev = cache.k_cache.device
    _need(q, "q", cache.dtype, 3, dev)
    _need(k, "k", cache.dtype, 3, dev)
    _need(v, "v", cache.dtype, 3, dev)
    _need(cu_chunk_lens, "cu_chunk_lens", torch.int32, 1, dev)
    _need(prefix_lens, "prefix_lens", torch.int32, 1, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    total, Hq, D = q.shape
    n = prefix_lens.shape[0]
    if cu_chunk_lens.shape[0] != n + 1 or block_table.shape[0] != n:
        raise ValueError("cu_chunk_lens / prefix_lens / block_table disagree on n_seqs")
    if k.shape != (total, cache.num_kv_heads, D) or v.shape != k.shape or D != cache.head_dim:
        raise ValueError("k / v must be [total_tokens, Hkv, head_dim]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", cache.dtype, 3, dev)
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    if max_context_len is None:
        _check("kvc_chunked_prefill_attention", LIB.kvc_chunked_prefill_attention(
            cache.c, q.data_ptr(), k.data_ptr(), v.data_ptr(), n, cu_chunk_lens.data_ptr(),
            prefix_lens.data_ptr(), total, int(max_chunk_len), block_table.data_ptr(),
            block_table.shape[1], Hq, scale, out.data_ptr(), _stream()))
        return out
    need = prefill_workspace_bytes(n, total, int(max_chunk_len), int(max_context_len), Hq,
                                   cache.num_kv_heads, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("kvc_chunked_prefill_attention_split", LIB.kvc_chunked_prefill_attention_split(
        cache.c, q.data_ptr(), k.data_ptr(), v.data_ptr(), n, cu_chunk_lens.data_ptr(),
        prefix_lens.data_ptr(), total, int(max_chunk_len), int(max_context_len),
        block_table.data_ptr(), block_table.shape[1], Hq, scale, out.data_ptr(),
        _ptr(workspace), ws_bytes, _stream()))
    return out


def mixed_workspace_bytes(n_decode: int, decode_max_context: int, Hq: int, num_kv_heads: int,
                          head_dim: int) -> int:
    return int(LIB.kvc_mixed_workspace_bytes(n_decode, decode_max_context, Hq, num_kv_heads,
                                             head_dim))


def mixed_step_attention(cache: PagedKVCache, Hq: int, *, q_decode=None, k_new=None, v_new=None,
                         decode_block_table=None, decode_context_lens=None,
                         decode_max_context: int = 0, q_prefill=None, k_prefill=None,
                         v_prefill=None, cu_chunk_lens=None, prefix_lens=None,
                         prefill_block_table=None, prefill_max_chunk: int = 0,
                         softmax_scale: float | None = None, out_decode=None, out_prefill=None,
                         workspace: torch.Tensor | None = None):
    """One mixed continuous-batching step in one launch (kvc_mixed_step_attention):
    decode rows as decode_append_attention takes them, prefill chunks as
    chunked_prefill_attention takes them. Returns (out_decode, out_prefill),
    either None when its part is empty. ``workspace`` must have its first 256
    bytes zero before the first call (each call leaves them zero); one of the
    size the library asks for is made with torch.zeros when none is given."""
    dev = cache.k_cache.device
    D = cache.head_dim
    b = _CMixed()
    if q_decode is not None and q_decode.shape[0] > 0:
        _need(q_decode, "q_decode", cache.dtype, 3, dev)
        n = q_decode.shape[0]
        if q_decode.shape != (n, Hq, D):
            raise ValueError(f"q_decode must be [{n}, {Hq}, {D}]")
        for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
            _need(t, nm, cache.dtype, 3, dev)
            if t.shape != (n, cache.num_kv_heads, D):
                raise ValueError(f"{nm} must be [{n}, {cache.num_kv_heads}, {D}]")
        _need(decode_block_table, "decode_block_table", torch.int32, 2, dev)
        _need(decode_context_lens, "decode_context_lens", torch.int32, 1, dev)
        if decode_block_table.shape[0] != n or decode_context_lens.shape[0] != n:
            raise ValueError("decode block table / context lengths disagree with q_decode")
        if out_decode is None:
            out_decode = torch.empty_like(q_decode)
        _need(out_decode, "out_decode", cache.dtype, 3, dev)
        if out_decode.shape != q_decode.shape:
            raise ValueError("out_decode must have q_decode's shape")
        b.n_decode, b.q_decode, b.k_new, b.v_new = n, q_decode.data_ptr(), k_new.data_ptr(), \
            v_new.data_ptr()
        b.decode_block_table, b.decode_max_blocks = decode_block_table.data_ptr(), \
            decode_block_table.shape[1]
        b.decode_context_lens, b.decode_max_context = decode_context_lens.data_ptr(), \
            int(decode_max_context)
        b.out_decode = out_decode.data_ptr()
    else:
        out_decode = None
    if q_prefill is not None and q_prefill.shape[0] > 0:
        _need(q_prefill, "q_prefill", cache.dtype, 3, dev)
        total = q_prefill.shape[0]
        if q_prefill.shape != (total, Hq, D):
            raise ValueError(f"q_prefill must be [{total}, {Hq}, {D}]")
        for t, nm in ((k_prefill, "k_prefill"), (v_prefill, "v_prefill")):
            _need(t, nm, cache.dtype, 3, dev)
            if t.shape != (total, cache.num_kv_heads, D):
                raise ValueError(f"{nm} must be [{total}, {cache.num_kv_heads}, {D}]")
        _need(cu_chunk_lens, "cu_chunk_lens", torch.int32, 1, dev)
        _need(prefix_lens, "prefix_lens", torch.int32, 1, dev)
        _need(prefill_block_table, "prefill_block_table", torch.int32, 2, dev)
        m = prefix_lens.shape[0]
        if cu_chunk_lens.shape[0] != m + 1 or prefill_block_table.shape[0] != m:
            raise ValueError("cu_chunk_lens / prefix_lens / prefill_block_table disagree")
        if out_prefill is None:
            out_prefill = torch.empty_like(q_prefill)
        _need(out_prefill, "out_prefill", cache.dtype, 3, dev)
        if out_prefill.shape != q_prefill.shape:
            raise ValueError("out_prefill must have q_prefill's shape")
        b.n_prefill, b.q_prefill = m, q_prefill.data_ptr()
        b.k_prefill, b.v_prefill = k_prefill.data_ptr(), v_prefill.data_ptr()
        b.cu_chunk_lens, b.prefix_lens = cu_chunk_lens.data_ptr(), prefix_lens.data_ptr()
        b.prefill_total_tokens, b.prefill_max_chunk = total, int(prefill_max_chunk)
        b.prefill_block_table, b.prefill_max_blocks = prefill_block_table.data_ptr(), \
            prefill_block_table.shape[1]
        b.out_prefill = out_prefill.data_ptr()
    else:
        out_prefill = None
    need = mixed_workspace_bytes(b.n_decode, b.decode_max_context, Hq, cache.num_kv_heads, D)
    if workspace is None:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    _check("kvc_mixed_step_attention", LIB.kvc_mixed_step_attention(
        cache.c, ctypes.byref(b), int(Hq), scale, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out_decode, out_prefill


def stream_read(data: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Streaming-read probe (kvc_stream_read): reads every byte of the contiguous
    GPU tensor `data` once. Returns int32 [kvc_stream_read_groups()] holding each
    workgroup's wrapping 32-bit sum of the words it read (as int32 bits)."""
    _need(data, "data")
    nbytes = data.numel() * data.element_size()
    groups = int(LIB.kvc_stream_read_groups())
    if out is None:
        out = torch.empty(groups, dtype=torch.int32, device=data.device)
    _need(out, "out", torch.int32, 1, data.device)
    if out.shape[0] != groups:
        raise ValueError(f"out must have {groups} entries")
    _check("kvc_stream_read", LIB.kvc_stream_read(data.data_ptr(), nbytes, out.data_ptr(),
                                                  _stream()))
    return out


KVC_ERR_NO_BLOCKS = -7


class PrefixCache:
    """Host-side block manager with prefix matching (include/kvc_prefix.h).

    Block ids index the first dimension of every layer's pool. ``match`` and
    ``allocate`` take references, ``release`` drops them, ``commit`` makes a
    sequence's full blocks matchable once their K/V are written."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        self._h = LIB.kvc_prefix_cache_create(int(num_blocks), int(block_size))
        if not self._h:
            raise KvcError("kvc_prefix_cache_create", -2, "bad pool shape or out of memory")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            LIB.kvc_prefix_cache_destroy(h)

    @staticmethod
    def _ints(xs):
        a = (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])
        return a

    def match(self, tokens, max_blocks: int | None = None) -> list[int]:
        toks = self._ints(tokens)
        cap = (len(tokens) // self.block_size) if max_blocks is None else int(max_blocks)
        out = (ctypes.c_int32 * max(1, cap))()
        n = LIB.kvc_prefix_cache_match(self._h, toks, len(tokens), out, cap)
        _check("kvc_prefix_cache_match", min(n, 0))
        return list(out[:n])

    def allocate(self, n: int) -> list[int] | None:
        """``n`` new blocks, or None when the pool cannot supply them."""
        out = (ctypes.c_int32 * max(1, n))()
        got = LIB.kvc_prefix_cache_allocate(self._h, int(n), out)
        if got == KVC_ERR_NO_BLOCKS:
            return None
        _check("kvc_prefix_cache_allocate", min(got, 0))
        return list(out[:n])

    def commit(self, tokens, block_ids) -> None:
        _check("kvc_prefix_cache_commit", LIB.kvc_prefix_cache_commit(
            self._h, self._ints(tokens), len(tokens), self._ints(block_ids), len(block_ids)))

    def release(self, block_ids) -> None:
        _check("kvc_prefix_cache_release", LIB.kvc_prefix_cache_release(
            self._h, self._ints(block_ids), len(block_ids)))

    def refcount(self, block_id: int) -> int:
        r = LIB.kvc_prefix_cache_refcount(self._h, int(block_id))
        _check("kvc_prefix_cache_refcount", min(r, 0))
        return r

    def counts(self) -> tuple[int, int, int]:
        """(free, cached, referenced) block counts."""
        f, c, r = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("kvc_prefix_cache_counts", LIB.kvc_prefix_cache_counts(
            self._h, ctypes.byref(f), ctypes.byref(c), ctypes.byref(r)))
        return f.value, c.value, r.value


SCHED_PREFILL_FIRST = 0
SCHED_DECODE_FIRST = 1
SCHED_STATIC = 2


@dataclasses.dataclass
class SchedStep:
    """One step built by :class:`Scheduler` (host int32 arrays)."""
    decode_ids: np.ndarray
    decode_context_lens: np.ndarray
    decode_block_table: np.ndarray     # [n_decode, max_blocks], unused columns -1
    decode_max_context: int
    prefill_ids: np.ndarray
    prefill_prefix_lens: np.ndarray
    prefill_cu_chunk_lens: np.ndarray  # [n_prefill + 1]
    prefill_block_table: np.ndarray    # [n_prefill, max_blocks]
    prefill_total_tokens: int
    prefill_max_chunk: int
    prefill_max_context: int
    first_token_ids: np.ndarray
    finished_ids: np.ndarray


class Scheduler:
    """Iteration-level scheduler and step builder (include/kvc_sched.h)."""

    def __init__(self, policy: int, slots: int, token_budget: int, num_blocks: int,
                 max_blocks_per_seq: int):
        self._h = LIB.kvc_sched_create(int(policy), int(slots), int(token_budget),
                                       int(num_blocks), int(max_blocks_per_seq))
        if not self._h:
            raise KvcError("kvc_sched_create", -2, "bad policy or sizes, or out of memory")
        self.slots, self.max_blocks = int(slots), int(max_blocks_per_seq)
        n, m = self.slots, self.max_blocks
        self._buf = {k: np.zeros(sz, np.int32) for k, sz in (
            ("decode_ids", n), ("decode_context_lens", n), ("decode_block_table", n * m),
            ("prefill_ids", n), ("prefill_prefix_lens", n), ("prefill_cu_chunk_lens", n + 1),
            ("prefill_block_table", n * m), ("first_token_ids", n), ("finished_ids", n))}
        self._c = _CStep(**{k: v.ctypes.data_as(_CStep._p) for k, v in self._buf.items()})

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            LIB.kvc_sched_destroy(h)

    def submit(self, prompt_len: int, answer_len: int) -> int:
        r = LIB.kvc_sched_submit(self._h, int(prompt_len), int(answer_len))
        _check("kvc_sched_submit", min(r, 0))
        return r

    def unfinished(self) -> int:
        return LIB.kvc_sched_unfinished(self._h)

    def next_step(self) -> SchedStep | None:
        """The next step, or None when nothing is queued or running. Raises
        KvcError (status KVC_ERR_NO_BLOCKS) when the pool cannot cover it."""
        r = LIB.kvc_sched_next_step(self._h, ctypes.byref(self._c))
        _check("kvc_sched_next_step", min(r, 0))
        if r == 0:
            return None
        c, b, m = self._c, self._buf, self.max_blocks
        nd, npf = c.n_decode, c.n_prefill
        return SchedStep(
            b["decode_ids"][:nd].copy(), b["decode_context_lens"][:nd].copy(),
            b["decode_block_table"][:nd * m].reshape(nd, m).copy(), c.decode_max_context,
            b["prefill_ids"][:npf].copy(), b["prefill_prefix_lens"][:npf].copy(),
            b["prefill_cu_chunk_lens"][:npf + 1].copy(),
            b["prefill_block_table"][:npf * m].reshape(npf, m).copy(),
            c.prefill_total_tokens, c.prefill_max_chunk, c.prefill_max_context,
            b["first_token_ids"][:c.n_first].copy(), b["finished_ids"][:c.n_finished].copy())
