"""Shared builders for the GPU parity tests.

Inputs come from `workloads` (seeded); the expected values come from `oracle`
only. The HIP side is driven through the kv_cache_decode_append_amd binding.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import workloads as W
from oracle import attention as OA
from oracle import bf16 as OB
from oracle import paged as OP

TDTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}
FILL = -1          # all-ones bit pattern: NaN sentinel in fp32 and bf16


def say(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def oracle_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cache-dtype values the oracle computes on (fp64 copy)."""
    if dtype == "bf16":
        return OB.round_bf16(x).astype(np.float64)
    return x.astype(np.float64)


def oracle_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return OB.to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Test-side input preparation: fp32 -> cache dtype on the CPU (RNE), then upload."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TDTYPE[dtype])
    return t.to(device)


def device_bits(t: torch.Tensor) -> np.ndarray:
    ib = torch.int16 if t.dtype == torch.bfloat16 else torch.int32
    a = t.contiguous().view(ib).cpu().numpy()
    return a.view(np.uint16 if t.dtype == torch.bfloat16 else np.uint32)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    if dtype == "fp32":
        assert err <= 1e-5, f"{what}: max abs err {err:.3e} > 1e-5"
    else:
        scale = float(np.max(np.abs(ref))) if ref.size else 1.0
        assert err <= 1e-2, f"{what}: max abs err {err:.3e} > 1e-2"
        assert err <= 2.0 ** -7 * scale, f"{what}: normalised err {err / scale:.3e} > 2^-7"
    return err


class DecodeCase:
    """One append + decode step for a batch of sequences of mixed lengths.

    ctx[b] counts the tokens held after the step, so the new token of sequence b
    sits at position ctx[b] - 1 and positions 0 .. ctx[b] - 2 are already cached.
    """

    def __init__(self, w: W.Workload, ctx, num_blocks: int, seed_extra: int = 0,
                 max_blocks: int | None = None, keep_host: bool = True):
        self.w = w
        self.ctx = np.asarray(ctx, dtype=np.int64)
        self.B = len(self.ctx)
        self.num_blocks = num_blocks
        self.bt = W.block_tables(w, self.ctx, num_blocks, max_blocks=max_blocks,
                                 seed_extra=seed_extra)
        self.k, self.v, self.q = [], [], np.empty((self.B, w.Hq, w.D), np.float32)
        for b, n in enumerate(self.ctx):
            k, v, q = W.sequence_values(w, b, int(n), 1)
            self.k.append(k)
            self.v.append(v)
            self.q[b] = q[0]

    # ---------------------------------------------------------------- oracle side
    def oracle_out(self, rows=None) -> np.ndarray:
        rows = range(self.B) if rows is None else rows
        dt = self.w.dtype
        scale = OA.default_scale(self.w.D)
        return np.stack([
            OA.attend_row(oracle_values(self.q[b], dt), oracle_values(self.k[b], dt),
                          oracle_values(self.v[b], dt), scale) if self.ctx[b] > 0
            else np.zeros((self.w.Hq, self.w.D)) for b in rows])

    def oracle_slots(self):
        seq, pos = self.token_lists()
        return OP.slots_for_positions(self.bt, seq, pos, W.BLOCK_SIZE)

    def oracle_pool(self):
        bits = 16 if self.w.dtype == "bf16" else 32
        pk = OP.empty_pool(self.num_blocks, self.w.Hkv, W.BLOCK_SIZE, self.w.D, bits)
        pv = pk.copy()
        slots = self.oracle_slots()
        off = 0
        for b, n in enumerate(self.ctx):
            n = int(n)
            OP.scatter(pk, slots[off:off + n], oracle_bits(self.k[b], self.w.dtype))
            OP.scatter(pv, slots[off:off + n], oracle_bits(self.v[b], self.w.dtype))
            off += n
        return pk, pv

    def token_lists(self):
        seq = np.concatenate([np.full(int(n), b, np.int64) for b, n in enumerate(self.ctx)])
        pos = np.concatenate([np.arange(int(n), dtype=np.int64) for n in self.ctx])
        return seq, pos

    # ---------------------------------------------------------------- GPU side
    def run_gpu(self, kvc, max_context_len: int | None = None, fused: bool = False):
        """Fill the cache through slot_mapping + kv_append (cached tokens, then
        the new ones), then decode; with `fused` the new tokens are appended by
        the decode launch itself (decode_append_attention, the launch the
        benchmark times). Returns (cache, out)."""
        w, dev = self.w, "cuda"
        cache = kvc.PagedKVCache.allocate(self.num_blocks, w.Hkv, w.D, TDTYPE[w.dtype],
                                          fill_bits=FILL)
        bt = torch.from_numpy(self.bt).to(dev)
        old = [b for b in range(self.B) if self.ctx[b] > 1]
        if old:
            seq = torch.from_numpy(np.concatenate(
                [np.full(int(self.ctx[b]) - 1, b, np.int32) for b in old])).to(dev)
            pos = torch.from_numpy(np.concatenate(
                [np.arange(int(self.ctx[b]) - 1, dtype=np.int32) for b in old])).to(dev)
            kk = to_device(np.concatenate([self.k[b][:-1] for b in old]), w.dtype)
            vv = to_device(np.concatenate([self.v[b][:-1] for b in old]), w.dtype)
            s_old = kvc.slot_mapping(bt, self.num_blocks, seq, pos, err_flag=cache.err_flag)
            kvc.kv_append(cache, s_old, kk, vv)
        live = [b for b in range(self.B) if self.ctx[b] > 0]
        if fused:
            assert len(live) == self.B, "the fused launch appends one token to every row"
            q = to_device(self.q, w.dtype)
            kn = to_device(np.stack([self.k[b][-1] for b in live]), w.dtype)
            vn = to_device(np.stack([self.v[b][-1] for b in live]), w.dtype)
            ctx = torch.from_numpy(self.ctx.astype(np.int32)).to(dev)
            mcl = int(self.ctx.max()) if max_context_len is None else max_context_len
            out = kvc.decode_append_attention(cache, q, kn, vn, bt, ctx, mcl)
            torch.cuda.synchronize()
            return cache, out
        if live:
            seq = torch.tensor(live, dtype=torch.int32, device=dev)
            pos = torch.tensor([int(self.ctx[b]) - 1 for b in live], dtype=torch.int32, device=dev)
            kn = to_device(np.stack([self.k[b][-1] for b in live]), w.dtype)
            vn = to_device(np.stack([self.v[b][-1] for b in live]), w.dtype)
            s_new = kvc.slot_mapping(bt, self.num_blocks, seq, pos, err_flag=cache.err_flag)
            kvc.kv_append(cache, s_new, kn, vn)
        q = to_device(self.q, w.dtype)
        ctx = torch.from_numpy(self.ctx.astype(np.int32)).to(dev)
        mcl = int(self.ctx.max()) if max_context_len is None else max_context_len
        out = kvc.paged_decode_attention(cache, q, bt, ctx, mcl)
        torch.cuda.synchronize()
        return cache, out


def max_rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def default_scale(d):
    return 1.0 / math.sqrt(d)


class PrefillCase:
    """Chunked prefill for a batch of sequences: sequence i already holds
    prefix[i] cached tokens and now writes + attends a chunk of chunk[i] tokens."""

    def __init__(self, w: W.Workload, prefix, chunk, num_blocks: int, seed_extra: int = 0):
        self.w = w
        self.prefix = np.asarray(prefix, dtype=np.int64)
        self.chunk = np.asarray(chunk, dtype=np.int64)
        self.n = len(self.prefix)
        self.total = self.prefix + self.chunk
        self.num_blocks = num_blocks
        self.bt = W.block_tables(w, self.total, num_blocks, seed_extra=seed_extra)
        self.k, self.v, self.q = [], [], []
        for i in range(self.n):
            k, v, q = W.sequence_values(w, i, int(self.total[i]), int(self.chunk[i]))
            self.k.append(k)
            self.v.append(v)
            self.q.append(q)

    def oracle_rows(self, i: int, rows=None) -> np.ndarray:
        dt = self.w.dtype
        q = oracle_values(self.q[i], dt)
        k = oracle_values(self.k[i], dt)
        v = oracle_values(self.v[i], dt)
        scale = OA.default_scale(self.w.D)
        p0 = int(self.prefix[i])
        if rows is None:
            return OA.prefill_chunk_rows(q, k, v, p0, scale)
        return np.stack([OA.attend_row(q[r], k[:p0 + r + 1], v[:p0 + r + 1], scale) for r in rows])

    def oracle_pool(self):
        bits = 16 if self.w.dtype == "bf16" else 32
        pk = OP.empty_pool(self.num_blocks, self.w.Hkv, W.BLOCK_SIZE, self.w.D, bits)
        pv = pk.copy()
        for i in range(self.n):
            n = int(self.total[i])
            slots = OP.slots_for_positions(self.bt, [i] * n, np.arange(n), W.BLOCK_SIZE)
            OP.scatter(pk, slots, oracle_bits(self.k[i], self.w.dtype))
            OP.scatter(pv, slots, oracle_bits(self.v[i], self.w.dtype))
        return pk, pv

    def run_gpu(self, kvc, cache=None, max_context_len=None):
        """Cache the prefixes through slot_mapping + kv_append, then one chunked
        prefill call for all sequences (the key-range split entry point when
        max_context_len is given). Returns (cache, out [sum C, Hq, D])."""
        w, dev = self.w, "cuda"
        if cache is None:
            cache = kvc.PagedKVCache.allocate(self.num_blocks, w.Hkv, w.D, TDTYPE[w.dtype],
                                              fill_bits=FILL)
        bt = torch.from_numpy(self.bt).to(dev)
        old = [i for i in range(self.n) if self.prefix[i] > 0]
        if old:
            seq = torch.from_numpy(np.concatenate(
                [np.full(int(self.prefix[i]), i, np.int32) for i in old])).to(dev)
            pos = torch.from_numpy(np.concatenate(
                [np.arange(int(self.prefix[i]), dtype=np.int32) for i in old])).to(dev)
            kk = to_device(np.concatenate([self.k[i][:self.prefix[i]] for i in old]), w.dtype)
            vv = to_device(np.concatenate([self.v[i][:self.prefix[i]] for i in old]), w.dtype)
            s = kvc.slot_mapping(bt, self.num_blocks, seq, pos, err_flag=cache.err_flag)
            kvc.kv_append(cache, s, kk, vv)
        cu = np.concatenate([[0], np.cumsum(self.chunk)]).astype(np.int32)
        q = to_device(np.concatenate(self.q), w.dtype)
        k = to_device(np.concatenate([self.k[i][self.prefix[i]:] for i in range(self.n)]), w.dtype)
        v = to_device(np.concatenate([self.v[i][self.prefix[i]:] for i in range(self.n)]), w.dtype)
        out = kvc.chunked_prefill_attention(
            cache, q, k, v, torch.from_numpy(cu).to(dev),
            torch.from_numpy(self.prefix.astype(np.int32)).to(dev), bt, int(self.chunk.max()),
            max_context_len=max_context_len)
        torch.cuda.synchronize()
        self.cu = cu
        return cache, out
