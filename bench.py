"""Decode-step benchmark on one MI355X: KV-read GB/s and batched decode steps/s.

Workload (Llama-3.1-8B attention shape, batch 64, context ~2k): 32 query heads,
8 KV heads, head_dim 128, bf16 cache, 16-token blocks, context lengths uniform
in [2000, 2300] counting the new token, one 9,200-block pool per layer for 32
layers (17.97 GiB of K/V in HBM, so repeated steps cannot be served from the
256 MB Infinity Cache). A step is one decode step of the whole model's
attention: slot mapping of the 64 new tokens, then for each of the 32 layers
kv_append of the new K/V and paged decode attention (with its split-K merge).
Inputs are synthetic and resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints ONE JSON line. `value` is KV bytes read per second over the whole step.
The `roofline` entry is for the decode-attention call (paged_decode_kernel +
decode_merge_kernel), timed with HIP events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import resource
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, public spec
LAYERS = 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    return ap.parse_args()


def cpu_baseline(budget_s: float):
    """The oracle (cached-row form) on the same workload's sequences, on the
    host cores: as many whole sequences of one layer as fit the time budget."""
    import workloads as W
    from oracle import attention as OA
    from oracle import bf16 as OB

    w = W.C3
    ctx = W.context_lengths(w)
    scale = OA.default_scale(w.D)
    done_bytes, n_seq = 0, 0
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t_run = 0.0
    for b in range(w.B):
        k, v, q = W.sequence_values(w, b, int(ctx[b]), 1)
        kq = OB.round_bf16(k).astype(np.float64)
        vq = OB.round_bf16(v).astype(np.float64)
        qq = OB.round_bf16(q[0]).astype(np.float64)
        t0 = time.perf_counter()
        OA.attend_row(qq, kq, vq, scale)
        t_run += time.perf_counter() - t0
        done_bytes += int(ctx[b]) * w.Hkv * w.D * 2 * 2
        n_seq += 1
        if t_run >= budget_s:
            break
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu_s = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    # naive recompute-everything loop, a few positions of one sequence
    k, v, q = W.sequence_values(w, 0, int(ctx[0]), int(ctx[0]))
    kq = OB.round_bf16(k).astype(np.float64)
    vq = OB.round_bf16(v).astype(np.float64)
    qq = OB.round_bf16(q).astype(np.float64)
    t0 = time.perf_counter()
    rows = 64
    OA.causal_rows(qq, kq, vq, int(ctx[0]) - rows, int(ctx[0]) - 1, scale)
    t_naive_rows = time.perf_counter() - t0
    naive_step_s = t_naive_rows / rows * int(ctx[0])     # one sequence's full recompute
    return {
        "value": round(done_bytes / t_run / 1e9, 4),
        "unit": "GB/s",
        "cores": max(1, round(cpu_s / max(t_run, 1e-9))),
        "cores_available": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"cached-row oracle (fp64 numpy) for {n_seq} of 64 sequences of one layer of "
                   f"the decode step, {done_bytes / 1e6:.1f} MB of KV in {t_run:.2f} s"),
        "naive_oracle_one_sequence_s_extrapolated": round(naive_step_s, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path needs no collectives and runs on a single MI355X)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.C3
    L = args.layers
    ctx_np = W.context_lengths(w)
    bt_np = W.block_tables(w, ctx_np, W.C3_POOL_BLOCKS)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    nb = W.C3_POOL_BLOCKS
    max_ctx = int(ctx_np.max())

    g = torch.Generator(device=dev)
    g.manual_seed(3)
    caches = []
    base = None
    for layer in range(L):
        c = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev)
        if base is None:
            c.k_cache.normal_(0.0, 0.5, generator=g)
            c.v_cache.normal_(0.0, 0.5, generator=g)
            base = c
        else:
            c.k_cache.copy_(base.k_cache)
            c.v_cache.copy_(base.v_cache)
        caches.append(c)
    q = [torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5, generator=g)
         for _ in range(L)]
    kn = [torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5, generator=g)
          for _ in range(L)]
    vn = [torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5, generator=g)
          for _ in range(L)]
    out = [torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    bt = torch.from_numpy(bt_np).to(dev)
    ctx = torch.from_numpy(ctx_np.astype(np.int32)).to(dev)
    seq_ids = torch.arange(B, dtype=torch.int32, device=dev)
    pos = (ctx - 1).to(torch.int32)
    slots = torch.empty(B, dtype=torch.int64, device=dev)
    ws = torch.empty(max(1, kvc.decode_workspace_bytes(B, Hq, D, max_ctx)), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        kvc.slot_mapping(bt, nb, seq_ids, pos, out=slots)
        for layer in range(L):
            kvc.kv_append(caches[layer], slots, kn[layer], vn[layer])
            if ev is not None:
                ev[layer][0].record()
            kvc.paged_decode_attention(caches[layer], q[layer], bt, ctx, max_ctx,
                                       out=out[layer], workspace=ws)
            if ev is not None:
                ev[layer][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    errs = [int(c.err_flag.item()) for c in caches]
    if any(errs) or not all(torch.isfinite(o.float()).all().item() for o in out):
        print(f"bench sanity check failed: err flags {errs}", file=sys.stderr)
        sys.exit(1)

    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(L)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(events[s])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    dec_ms = np.array([[e[0].elapsed_time(e[1]) for e in st] for st in events])

    kv_bytes_layer = int(ctx_np.sum()) * Hkv * D * 2 * 2
    io_bytes_layer = (B * Hq * D * 2 * 2            # q in, out
                      + B * bt_np.shape[1] * 4 + B * 4)   # block table, context lengths
    kv_gbs = kv_bytes_layer * L / (ms_per_step * 1e-3) / 1e9
    dec_avg_us = float(dec_ms.mean() * 1e3)
    achieved = (kv_bytes_layer + io_bytes_layer) / (dec_avg_us * 1e-6) / 1e9

    res = {
        "metric": "decode-attn KV-read GB/s (% of HBM peak) + batched decode steps/s, B=64 ctx~2k",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "decode_steps_per_s": round(1000.0 / ms_per_step, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "llama3.1-8b attention decode, B=64, ctx U[2000,2300], GQA 32/8, "
                        "head_dim 128, bf16 paged cache (16-token blocks), 32 layers",
            "B": B, "Hq": Hq, "Hkv": Hkv, "head_dim": D, "block_size": 16, "layers": L,
            "ctx_sum": int(ctx_np.sum()), "pool_blocks_per_layer": nb,
            "kv_bytes_per_layer": kv_bytes_layer,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_kernel + decode_merge_kernel (one decode-attention call)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_us": round(dec_avg_us, 2),
            "bytes_per_launch": kv_bytes_layer + io_bytes_layer,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_budget_s)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
