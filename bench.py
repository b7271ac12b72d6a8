"""Decode-step benchmark on one MI355X: KV-read GB/s and batched decode steps/s.

Workload (Llama-3.1-8B attention shape, batch 64, context ~2k): 32 query heads,
8 KV heads, head_dim 128, bf16 cache, 16-token blocks, context lengths uniform
in [2000, 2300] counting the new token, one 9,200-block pool per layer for 32
layers (17.97 GiB of K/V in HBM, so repeated steps cannot be served from the
256 MB Infinity Cache). A step is one decode step of the whole model's
attention: for each of the 32 layers one fused launch that computes the 64 new
tokens' slots, appends their K/V to the paged cache and runs paged decode
attention (split-K merge pass only when a sequence spans several partitions).
Inputs are synthetic and resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload c3-decode|c3-fp8|c3-tp8-share|c4-mixed|c4-mixed-fp8|
                                c5-decode|c5-prefill|c5-prefill-fp8|prefix-warm|queue-replay]

The default workload is the one above (c3-decode). c5-decode (8 sequences at
32,000 tokens, split-K) and c5-prefill (8 x a 2,048-token chunk over a
30,000-token cached prefix, MFMA) measure the other kernels of the path on the
long-context workload; each prints its own line with its own roofline.
c3-tp8-share runs one GPU's share of the default step when the 8 kv heads are
spread over 8 GPUs (one kv head and its 4 query heads per layer, same kernel).

Prints ONE JSON line. `value` is KV bytes read per second over the whole step.
The `roofline` entry is for the per-layer decode launch (paged_decode_kernel,
with the append fused in): the timed region is nothing but those launches,
back to back on one stream between two HIP events.
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
    ap.add_argument("--workload", default="c3-decode",
                    choices=["c3-decode", "c3-fp8", "c3-tp8-share", "c4-mixed", "c4-mixed-fp8",
                             "c5-decode", "c5-prefill",
                             "c5-prefill-fp8", "prefix-warm", "queue-replay"])
    ap.add_argument("--direct-steps", type=int, default=400,
                    help="queue-replay: leading steps of each continuous plan run for real")
    return ap.parse_args()


# Files the decode kernel is compiled from; the traffic figure is only valid
# for the exact sources the counters were taken on.
DECODE_SOURCES = ("kv_cache_decode_append_amd/csrc/kvc_decode.hip",
                  "kv_cache_decode_append_amd/csrc/kvc_decode_item.h",
                  "kv_cache_decode_append_amd/csrc/kvc_device.h",
                  "kv_cache_decode_append_amd/csrc/kvc_host.h",
                  "include/kvc.h")


def sources_sha256(paths) -> str:
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(summary: str, sources=DECODE_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (profiles/), or None once any source of the kernel differs from
    the ones the counters were taken on."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", summary)) as f:
            rec = json.load(f)
        sha = sources_sha256(sources)
    except (OSError, ValueError):
        return None
    return rec.get("traffic_bytes_per_dispatch") if rec.get("kernel_sources_sha256") == sha else None


def cpu_baseline(budget_s: float):
    """The oracle (cached-row form) on the same workload: whole decode steps
    (64 sequences x 32 layers; the layers reuse one set of values, which does
    not change the oracle's work) on the host cores until the time budget is
    spent, at least one step."""
    import workloads as W
    from oracle import attention as OA
    from oracle import bf16 as OB

    w = W.C3
    ctx = W.context_lengths(w)
    scale = OA.default_scale(w.D)
    seqs = []
    for b in range(w.B):
        k, v, q = W.sequence_values(w, b, int(ctx[b]), 1)
        seqs.append((OB.round_bf16(q[0]).astype(np.float64), OB.round_bf16(k).astype(np.float64),
                     OB.round_bf16(v).astype(np.float64)))
    step_bytes = int(ctx.sum()) * w.Hkv * w.D * 2 * 2 * LAYERS
    done_bytes, n_steps = 0, 0
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t_run = 0.0
    while n_steps == 0 or t_run < budget_s:
        t0 = time.perf_counter()
        for _layer in range(LAYERS):
            for qq, kq, vq in seqs:
                OA.attend_row(qq, kq, vq, scale)
        t_run += time.perf_counter() - t0
        done_bytes += step_bytes
        n_steps += 1
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu_s = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    # naive recompute-everything loop at C3: the last 64 rows of one sequence's
    # full causal attention, timed; row i costs in proportion to its i + 1 keys,
    # so the whole recompute of a sequence of n tokens costs n(n+1)/2 such units
    n0 = int(ctx[0])
    k, v, q = W.sequence_values(w, 0, n0, n0)
    kq = OB.round_bf16(k).astype(np.float64)
    vq = OB.round_bf16(v).astype(np.float64)
    qq = OB.round_bf16(q).astype(np.float64)
    rows = 64
    t0 = time.perf_counter()
    OA.causal_rows(qq, kq, vq, n0 - rows, n0 - 1, scale)
    per_unit = (time.perf_counter() - t0) / sum(i + 1 for i in range(n0 - rows, n0))
    naive_seq_s = per_unit * n0 * (n0 + 1) / 2
    naive_layer_s = per_unit * float(sum(int(c) * (int(c) + 1) / 2 for c in ctx))
    # the naive and the cached loop over all of the fp32 toy (prompt 16, answer 48)
    w1 = W.C1
    n1 = W.C1_PROMPT + W.C1_ANSWER
    k1, v1, q1 = W.sequence_values(w1, 0, n1, n1)
    s1 = OA.default_scale(w1.D)
    t0 = time.perf_counter()
    OA.generate_uncached(q1, k1, v1, W.C1_PROMPT, W.C1_ANSWER, s1)
    c1_naive_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    OA.generate_cached(q1, k1, v1, W.C1_PROMPT, W.C1_ANSWER, s1)
    c1_cached_s = time.perf_counter() - t0
    try:
        import threadpoolctl
        blas_threads = max((i.get("num_threads", 0) for i in threadpoolctl.threadpool_info()
                            if i.get("user_api") == "blas"), default=None)
    except ImportError:
        blas_threads = None
    return {
        "value": round(done_bytes / t_run / 1e9, 4),
        "unit": "GB/s",
        "cores": max(1, round(cpu_s / max(t_run, 1e-9))),
        "cores_available": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"cached-row oracle (fp64 numpy), {n_steps} whole decode steps (64 sequences x "
                   f"{LAYERS} layers), {done_bytes / 1e9:.1f} GB of KV in {t_run:.1f} s"),
        "steps_per_s": round(n_steps / t_run, 4),
        "blas_threads": blas_threads,
        "naive_c3_one_sequence_s_extrapolated": round(naive_seq_s, 2),
        "naive_c3_layer_64_sequences_s_extrapolated": round(naive_layer_s, 1),
        "naive_extrapolation": (f"timed: rows {n0 - rows}..{n0 - 1} of sequence 0 (ctx {n0}); "
                                "scaled by the keys each row of the full recompute sees"),
        "c1_naive_loop_s": round(c1_naive_s, 4),
        "c1_cached_loop_s": round(c1_cached_s, 4),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path needs no collectives and runs on a single MI355X)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload == "c5-decode":
        return bench_c5_decode(args)
    if args.workload == "c5-prefill":
        return bench_c5_prefill(args)
    if args.workload == "c5-prefill-fp8":
        return bench_c5_prefill(args, fp8=True)
    if args.workload == "prefix-warm":
        return bench_prefix_warm(args)
    if args.workload == "c4-mixed":
        return bench_c4_mixed(args)
    if args.workload == "c4-mixed-fp8":
        return bench_c4_mixed(args, fp8=True)
    if args.workload == "queue-replay":
        return bench_queue_replay(args)
    if args.workload == "c3-fp8":
        return bench_c3_fp8(args)
    if args.workload == "c3-tp8-share":
        return bench_c3_tp8_share(args)

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
    ws = torch.empty(max(1, kvc.decode_workspace_bytes(B, Hq, D, max_ctx)), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step():
        for layer in range(L):
            kvc.decode_append_attention(caches[layer], q[layer], kn[layer], vn[layer], bt, ctx,
                                        max_ctx, out=out[layer], workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    errs = [int(c.err_flag.item()) for c in caches]
    if any(errs) or not all(torch.isfinite(o.float()).all().item() for o in out):
        print(f"bench sanity check failed: err flags {errs}", file=sys.stderr)
        sys.exit(1)

    # The timed region is steps x 32 back-to-back launches of the decode kernel
    # on torch's current stream, bracketed by two HIP events on that stream;
    # the per-launch average is the region's time over the launch count.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # one more event after every step gives the per-step spread (a timestamp on
    # the stream between steps; the total is still start to end)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step()
        marks[i].record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per_step = np.array([t_start.elapsed_time(marks[0])]
                        + [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)])

    ceiling = read_ceiling_gbs(kvc, torch, dev)     # after the timed region

    kv_bytes_layer = int(ctx_np.sum()) * Hkv * D * 2 * 2
    io_bytes_layer = (B * Hq * D * 2 * 2            # q in, out
                      + B * Hkv * D * 2 * 2 * 2     # new K/V read and written to the cache
                      + B * bt_np.shape[1] * 4 + B * 4)   # block table, context lengths
    kv_gbs = kv_bytes_layer * L / (ms_per_step * 1e-3) / 1e9
    dec_avg_us = ms_per_step * 1e3 / L
    achieved = (kv_bytes_layer + io_bytes_layer) / (dec_avg_us * 1e-6) / 1e9

    res = {
        "metric": "decode-attn KV-read GB/s (% of HBM peak) + batched decode steps/s, B=64 ctx~2k",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "read_ceiling_gbs": round(ceiling, 1),
        "pct_read_ceiling": round(100.0 * kv_gbs / ceiling, 2),
        "decode_steps_per_s": round(1000.0 / ms_per_step, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_p10": round(float(np.percentile(per_step, 10)), 4),
        "step_ms_p90": round(float(np.percentile(per_step, 90)), 4),
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
            "kernel": "paged_decode_kernel (fused append + decode attention, one launch per layer)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_c3_counters.json"),
            "avg_us": round(dec_avg_us, 2),
            "bytes_per_launch": kv_bytes_layer + io_bytes_layer,
            "measured_read_ceiling": round(ceiling, 1),
            "frac_of_measured_ceiling": round(achieved / ceiling, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_budget_s)
    print(json.dumps(res), flush=True)


def bench_c3_fp8(args):
    """The C3 decode step over an fp8 (E4M3, one fp32 scale per token and kv
    head) cache: same batch, contexts, pools and launch pattern as the default
    workload, K/V codes and scales instead of bf16 values. KV bytes per token
    and kv head: 2 x (head_dim + 4). Queries, new K/V and outputs stay bf16."""
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
    for layer in range(L):
        c = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.float8_e4m3fn, device=dev)
        fill_fp8_pools(c, g)
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
    ws = torch.empty(max(1, kvc.decode_workspace_bytes(B, Hq, D, max_ctx)), dtype=torch.uint8,
                     device=dev)

    def step(i):
        for layer in range(L):
            kvc.decode_append_attention(caches[layer], q[layer], kn[layer], vn[layer], bt, ctx,
                                        max_ctx, out=out[layer], workspace=ws)

    ms_per_step = _timed(step, args.steps, args.warmup)
    errs = [int(c.err_flag.item()) for c in caches]
    if any(errs) or not all(torch.isfinite(o.float()).all().item() for o in out):
        print(f"bench sanity check failed: err flags {errs}", file=sys.stderr)
        sys.exit(1)
    kv_bytes_layer = int(ctx_np.sum()) * Hkv * (D + 4) * 2
    io_bytes_layer = (B * Hq * D * 2 * 2 + B * Hkv * D * 2 * 2 + B * Hkv * (D + 4) * 2
                      + B * bt_np.shape[1] * 4 + B * 4)
    kv_gbs = kv_bytes_layer * L / (ms_per_step * 1e-3) / 1e9
    avg_us = ms_per_step * 1e3 / L
    achieved = (kv_bytes_layer + io_bytes_layer) / (avg_us * 1e-6) / 1e9
    res = _base_line(args, "decode-attn KV-read GB/s + batched decode steps/s, B=64 ctx~2k, fp8 "
                     "E4M3 cache (per-row scales)", round(kv_gbs, 1), "GB/s", ms_per_step,
                     "fp8-e4m3 cache, bf16 compute",
                     {"workload": "llama3.1-8b attention decode, B=64, ctx U[2000,2300], GQA 32/8, "
                                  "head_dim 128, fp8 E4M3 paged cache with one fp32 scale per "
                                  "token and kv head, 32 layers",
                      "B": B, "layers": L, "ctx_sum": int(ctx_np.sum()),
                      "kv_bytes_per_layer": kv_bytes_layer},
                     {"bound": "hbm", "kernel": "paged_decode_kernel<fp8> (fused quantising "
                      "append + decode attention, one launch per layer)",
                      "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                      "avg_us": round(avg_us, 2), "bytes_per_launch": kv_bytes_layer + io_bytes_layer})
    res["pct_hbm_peak"] = round(100.0 * kv_gbs / HBM_PEAK_GBS, 2)
    res["decode_steps_per_s"] = round(1000.0 / ms_per_step, 2)
    print(json.dumps(res), flush=True)


def _timed(fn, steps, warmup):
    """Mean milliseconds per call over `steps` calls, HIP events on torch's stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def read_ceiling_gbs(kvc, torch, dev, gib=4, reps=10):
    """HBM read ceiling of this machine: the library's streaming-read probe
    (128-bit non-temporal loads, front to back) over a `gib` GiB buffer, 16x
    the 256 MB Infinity Cache, so every byte comes from HBM."""
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = kvc.stream_read(buf)
    for _ in range(3):
        kvc.stream_read(buf, out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        kvc.stream_read(buf, out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del buf, out
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def _base_line(args, metric, value, unit, ms, dtype, config, roofline):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "accumulate": "fp32",
            "data": "synthetic", "config": config, "roofline": roofline, "cpu_baseline": None}


def bench_c5_decode(args):
    """8 sequences x 32,000 tokens, GQA 32/8/128 bf16, fused append + split-K decode.
    Eight layer pools (2.1 GB each) are rotated so the Infinity Cache cannot hold them."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.C5
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    ctx_np = W.context_lengths(w)
    nb = B * W.blocks_for(W.C5_CTX)
    bt = torch.from_numpy(W.block_tables(w, ctx_np, nb)).to(dev)
    ctx = torch.from_numpy(ctx_np.astype(np.int32)).to(dev)
    L = 8
    caches = []
    for _ in range(L):
        c = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev)
        c.k_cache.normal_(0, 0.5)
        c.v_cache.normal_(0, 0.5)
        caches.append(c)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    kn = torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    vn = torch.empty_like(kn)
    out = torch.empty_like(q)
    ws = torch.empty(kvc.decode_workspace_bytes(B, Hq, D, W.C5_CTX), dtype=torch.uint8, device=dev)
    ms = _timed(lambda i: kvc.decode_append_attention(caches[i % L], q, kn, vn, bt, ctx, W.C5_CTX,
                                                      out=out, workspace=ws),
                args.steps, args.warmup)
    kv = int(ctx_np.sum()) * Hkv * D * 2 * 2
    gbs = kv / (ms * 1e-3) / 1e9
    res = _base_line(args, "long-context decode KV-read GB/s, B=8 ctx 32k", round(gbs, 1), "GB/s",
                     ms, "bf16",
                     {"workload": "decode B=8 ctx 32,000, GQA 32/8, head_dim 128, bf16 paged cache, "
                                  "split-K + merge", "B": B, "ctx": W.C5_CTX},
                     {"bound": "hbm", "kernel": "paged_decode_kernel + decode_merge_kernel",
                      "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                      "avg_us": round(ms * 1e3, 2), "bytes_per_launch": kv})
    print(json.dumps(res), flush=True)


def bench_c3_tp8_share(args):
    """One GPU's share of the default step under 8-way kv-head tensor
    parallelism: the same 64 sequences and context lengths, one kv head and its
    4 query heads per layer (the other kv heads sit on other GPUs; attention
    exchanges nothing). Same fused append + decode launch, split over keys as
    the library decides; 32 layer pools rotated."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.C3
    B, Hq, Hkv, D = w.B, w.Hq // 8, w.Hkv // 8, w.D
    L = args.layers
    ctx_np = W.context_lengths(w)
    nb = W.C3_POOL_BLOCKS
    bt = torch.from_numpy(W.block_tables(w, ctx_np, nb)).to(dev)
    ctx = torch.from_numpy(ctx_np.astype(np.int32)).to(dev)
    max_ctx = int(ctx_np.max())
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    caches = []
    for _ in range(L):
        c = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev)
        c.k_cache.normal_(0.0, 0.5, generator=g)
        c.v_cache.normal_(0.0, 0.5, generator=g)
        caches.append(c)
    mk = lambda h: torch.empty(B, h, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5, generator=g)
    q, kn, vn = mk(Hq), mk(Hkv), mk(Hkv)
    out = torch.empty_like(q)
    ws = torch.empty(max(1, kvc.decode_workspace_bytes(B, Hq, D, max_ctx)), dtype=torch.uint8,
                     device=dev)
    ms = _timed(lambda i: kvc.decode_append_attention(caches[i % L], q, kn, vn, bt, ctx, max_ctx,
                                                      out=out, workspace=ws),
                args.steps * L, args.warmup * L)
    errs = [int(c.err_flag.item()) for c in caches]
    if any(errs) or not torch.isfinite(out.float()).all().item():
        print(f"bench sanity check failed: err flags {errs}", file=sys.stderr)
        sys.exit(1)
    kv = int(ctx_np.sum()) * Hkv * D * 2 * 2
    # K/V, q, out, the new rows (read and written), block table and lengths
    per_launch = kv + 2 * B * Hq * D * 2 + 2 * 2 * B * Hkv * D * 2 + bt.numel() * 4 + B * 4
    step_ms = ms * L
    gbs = kv * L / (step_ms * 1e-3) / 1e9
    ach = per_launch / (ms * 1e-3) / 1e9
    res = _base_line(args, "decode KV-read GB/s, one GPU's share of the B=64 ctx~2k step under "
                     "kv-head tensor parallelism x8", round(gbs, 1), "GB/s", step_ms, "bf16",
                     {"workload": "B=64, ctx U[2000,2300], Hq 4 / Hkv 1 (one of 8 kv heads), "
                                  "head_dim 128, bf16 paged cache, 32 layers",
                      "B": B, "Hq": Hq, "Hkv": Hkv, "head_dim": D, "layers": L,
                      "split_workspace_bytes": kvc.decode_workspace_bytes(B, Hq, D, max_ctx)},
                     {"bound": "hbm", "kernel": "paged_decode_kernel (+ decode_merge_kernel when "
                      "split)", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                      "avg_us": round(ms * 1e3, 2), "bytes_per_launch": per_launch})
    res["decode_steps_per_s"] = round(1e3 / step_ms, 2)
    print(json.dumps(res), flush=True)


def fill_fp8_pools(cache, g=None):
    """Finite random E4M3 codes and row scales (about unit-sized values)."""
    import torch
    for pool in (cache.k_cache, cache.v_cache):
        code = torch.randint(0, 0x7F, pool.shape, generator=g, device=pool.device, dtype=torch.int32)
        sign = torch.randint(0, 2, pool.shape, generator=g, device=pool.device, dtype=torch.int32)
        pool.view(torch.uint8).copy_((code | (sign << 7)).to(torch.uint8))
    cache.k_scale.uniform_(0.5 / 448, 2.0 / 448, generator=g)
    cache.v_scale.uniform_(0.5 / 448, 2.0 / 448, generator=g)


def bench_c5_prefill(args, fp8=False):
    """8 sequences, each a 2,048-token chunk over a 30,000-token cached prefix
    (chunk K/V write + causal attention on MFMA). Algorithmic work counts only
    unmasked (query, key) pairs at 4 * head_dim flop each. With fp8 the cache
    holds E4M3 codes and row scales (dequantised to bf16 as tiles are staged)."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.C5
    n, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    P, C = W.C5_PREFIX, W.C5_CHUNK
    total = np.full(n, P + C)
    nb = n * W.blocks_for(P + C)
    bt = torch.from_numpy(W.block_tables(w, total, nb)).to(dev)
    if fp8:
        cache = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.float8_e4m3fn, device=dev)
        fill_fp8_pools(cache)
    else:
        cache = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev)
        cache.k_cache.normal_(0, 0.5)
        cache.v_cache.normal_(0, 0.5)
    q = torch.empty(n * C, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    k = torch.empty(n * C, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    cu = torch.arange(0, (n + 1) * C, C, dtype=torch.int32, device=dev)
    pre = torch.full((n,), P, dtype=torch.int32, device=dev)
    steps = max(1, args.steps // 10)
    ms = _timed(lambda i: kvc.chunked_prefill_attention(cache, q, k, v, cu, pre, bt, C, out=out),
                steps, max(1, args.warmup // 10))
    pairs = n * Hq * (C * P + C * (C + 1) // 2)
    flop = pairs * 4 * D
    tf = flop / (ms * 1e-3) / 1e12
    tag = ", fp8 E4M3 cache" if fp8 else ""
    res = _base_line(args, "chunked-prefill attention TFLOP/s, 8 x 2,048 over a 30,000 prefix" + tag,
                     round(tf, 1), "TFLOP/s", ms, "fp8-e4m3 cache, bf16 compute" if fp8 else "bf16",
                     {"workload": "chunked prefill, 8 sequences x 2,048-token chunk over a "
                                  "30,000-token cached prefix, GQA 32/8, head_dim 128, "
                                  + ("fp8 E4M3 cache with row scales" if fp8 else "bf16"),
                      "n_seqs": n, "chunk": C, "prefix": P},
                     {"bound": "mfma", "kernel": "chunk_append_kernel + prefill_attention_kernel",
                      "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                      "frac": round(tf / 2500.0, 4), "traffic": None,
                      "avg_us": round(ms * 1e3, 1), "flop_per_launch": flop})
    res["steps"] = steps
    print(json.dumps(res), flush=True)


def bench_c4_mixed(args, fp8=False):
    """The skewed continuous-batching step: 210 sequences with lognormal context
    lengths (median 6,000, tail clipped at 32,000); 206 decode one token each
    (one fused append + attention launch, split over partitions for the long
    ones) and 4 run a 2,048-token prefill chunk over their prefix (one launch).
    The same step is also timed as ONE launch of the mixed-batch kernel. One
    layer's pool (~6.5 GB, far larger than the caches) is timed per step and
    reported per layer and for 32 layers. With fp8 the cache holds E4M3 codes
    and one fp32 scale per (token, kv head) row for K and for V; the decode
    bytes count both."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.C4
    Hq, Hkv, D, L = w.Hq, w.Hkv, w.D, 32
    ctx = W.context_lengths(w)
    pre_rows = W.c4_prefill_rows(ctx)
    dec_rows = np.array([b for b in range(w.B) if b not in set(pre_rows.tolist())])
    need = int(sum(W.blocks_for(int(c)) for c in ctx))
    nb = need + need // 100
    bt_all = torch.from_numpy(W.block_tables(w, ctx, nb)).to(dev)
    if fp8:
        cache = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.float8_e4m3fn, device=dev)
        fill_fp8_pools(cache)
    else:
        cache = kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev)
        cache.k_cache.normal_(0, 0.5)
        cache.v_cache.normal_(0, 0.5)
    nd, chunk = len(dec_rows), W.C4_CHUNK
    q_dec = torch.empty(nd, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    k_dec = torch.empty(nd, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    v_dec = torch.empty_like(k_dec).normal_(0, 0.5)
    bt_dec = bt_all.index_select(0, torch.from_numpy(dec_rows.astype(np.int64)).to(dev)).contiguous()
    ctx_dec = torch.from_numpy(ctx[dec_rows].astype(np.int32)).to(dev)
    max_dec = int(ctx[dec_rows].max())
    ws = torch.empty(max(1, kvc.decode_workspace_bytes(nd, Hq, D, max_dec)), dtype=torch.uint8,
                     device=dev)
    out_dec = torch.empty_like(q_dec)
    npre = len(pre_rows)
    q_pre = torch.empty(npre * chunk, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    k_pre = torch.empty(npre * chunk, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    v_pre = torch.empty_like(k_pre).normal_(0, 0.5)
    out_pre = torch.empty_like(q_pre)
    cu = torch.arange(0, (npre + 1) * chunk, chunk, dtype=torch.int32, device=dev)
    prefix = torch.from_numpy((ctx[pre_rows] - chunk).astype(np.int32)).to(dev)
    bt_pre = bt_all.index_select(0, torch.from_numpy(pre_rows.astype(np.int64)).to(dev)).contiguous()

    def dec(i):
        kvc.decode_append_attention(cache, q_dec, k_dec, v_dec, bt_dec, ctx_dec, max_dec,
                                    out=out_dec, workspace=ws)

    def pre(i):
        kvc.chunked_prefill_attention(cache, q_pre, k_pre, v_pre, cu, prefix, bt_pre, chunk,
                                      out=out_pre)

    def step(i):
        dec(i)
        pre(i)

    mws = torch.zeros(kvc.mixed_workspace_bytes(nd, max_dec, Hq, Hkv, D), dtype=torch.uint8,
                      device=dev)

    def one_launch(i):
        kvc.mixed_step_attention(
            cache, Hq, q_decode=q_dec, k_new=k_dec, v_new=v_dec, decode_block_table=bt_dec,
            decode_context_lens=ctx_dec, decode_max_context=max_dec, q_prefill=q_pre,
            k_prefill=k_pre, v_prefill=v_pre, cu_chunk_lens=cu, prefix_lens=prefix,
            prefill_block_table=bt_pre, prefill_max_chunk=chunk, out_decode=out_dec,
            out_prefill=out_pre, workspace=mws)

    ms_dec = _timed(dec, args.steps, args.warmup)
    ms_pre = _timed(pre, max(1, args.steps // 4), max(1, args.warmup // 4))
    ms_step = _timed(step, max(1, args.steps // 4), max(1, args.warmup // 4))
    ms_one = _timed(one_launch, max(1, args.steps // 4), max(1, args.warmup // 4))

    def one_launch_dec(i):
        kvc.mixed_step_attention(
            cache, Hq, q_decode=q_dec, k_new=k_dec, v_new=v_dec, decode_block_table=bt_dec,
            decode_context_lens=ctx_dec, decode_max_context=max_dec, out_decode=out_dec,
            workspace=mws)

    def one_launch_pre(i):
        kvc.mixed_step_attention(
            cache, Hq, q_prefill=q_pre, k_prefill=k_pre, v_prefill=v_pre, cu_chunk_lens=cu,
            prefix_lens=prefix, prefill_block_table=bt_pre, prefill_max_chunk=chunk,
            out_prefill=out_pre, workspace=mws)

    ms_one_dec = _timed(one_launch_dec, max(1, args.steps // 4), max(1, args.warmup // 4))
    ms_one_pre = _timed(one_launch_pre, max(1, args.steps // 4), max(1, args.warmup // 4))
    # the caller-side route rule (StepRunner, auto): time both routes on this
    # step's size class, then report the route it keeps
    runner = kvc.StepRunner(Hq, trials=3)
    dec_part = dict(q=q_dec, k_new=k_dec, v_new=v_dec, block_table=bt_dec, context_lens=ctx_dec,
                    max_context=max_dec)
    pf_part = dict(q=q_pre, k=k_pre, v=v_pre, cu_chunk_lens=cu, prefix_lens=prefix,
                   block_table=bt_pre, max_chunk=chunk)
    for _ in range(8):
        runner.run(cache, dec_part, pf_part)
    torch.cuda.synchronize()
    route_key = runner.size_class(nd, max_dec, npre * chunk)
    assert int(cache.err_flag.item()) == 0
    assert int(mws[:256].count_nonzero().item()) == 0
    # K and V per token and kv head: bf16 values, or fp8 codes plus two fp32 row scales
    kv_dec = int(ctx[dec_rows].sum()) * Hkv * ((D + 4) * 2 if fp8 else D * 2 * 2)
    pairs = sum(Hq * (chunk * (int(c) - chunk) + chunk * (chunk + 1) // 2) for c in ctx[pre_rows])
    flop = pairs * 4 * D
    gbs = kv_dec / (ms_dec * 1e-3) / 1e9
    tf = flop / (ms_pre * 1e-3) / 1e12
    res = _base_line(args, "skewed mixed step (206 decode rows + 4 prefill chunks): decode KV-read "
                     "GB/s" + (", fp8 E4M3 cache" if fp8 else ""), round(gbs, 1), "GB/s", ms_step,
                     "fp8-e4m3 cache, bf16 compute" if fp8 else "bf16",
                     {"workload": "210 sequences, lognormal context (median 6,000, clipped at "
                                  "32,000), 206 decode + 4 x 2,048-token prefill chunks, GQA "
                                  "32/8, head_dim 128, "
                                  + ("fp8 E4M3 cache with row scales" if fp8 else "bf16")
                                  + ", one layer timed",
                      "B": int(w.B), "ctx_sum": int(ctx.sum()), "ctx_max": int(ctx.max()),
                      "prefill_rows": pre_rows.tolist(), "pool_blocks": nb},
                     {"bound": "hbm", "kernel": "paged_decode_kernel + decode_merge_kernel",
                      "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                      "avg_us": round(ms_dec * 1e3, 2), "bytes_per_launch": kv_dec})
    res["decode_ms_per_layer"] = round(ms_dec, 4)
    res["prefill_ms_per_layer"] = round(ms_pre, 4)
    res["step_ms_per_layer"] = round(ms_step, 4)
    res["step_ms_32_layers"] = round(ms_step * L, 3)
    res["one_launch_step_ms_per_layer"] = round(ms_one, 4)
    res["one_launch_step_ms_32_layers"] = round(ms_one * L, 3)
    res["one_launch_speedup"] = round(ms_step / ms_one, 3)
    res["one_launch_decode_only_ms"] = round(ms_one_dec, 4)
    res["one_launch_prefill_only_ms"] = round(ms_one_pre, 4)
    res["step_route"] = {"chosen": runner.decisions.get(route_key),
                         "separate_ms": [round(x, 4) for x in runner.samples[route_key]["separate"]],
                         "one_launch_ms": [round(x, 4) for x in
                                           runner.samples[route_key]["one_launch"]]}
    res["prefill_tflops"] = round(tf, 1)
    res["prefill_mfma_frac"] = round(tf / 2500.0, 4)
    print(json.dumps(res), flush=True)


def bench_prefix_warm(args):
    """Prefix caching at the Llama-3.1-8B attention shape: a 2,000-token prompt
    whose first 1,800 tokens are already cached. Cold = chunked prefill of all
    2,000 tokens; warm = block match in the native manager, then prefill of the
    208 tokens after the 112 cached blocks (1,792 tokens). Each is one launch
    per layer over 32 layer pools (the key-range split entry point, which
    spreads the few query tiles' keys over more workgroups; the plain call is
    timed too); the match is timed on the host."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.P1
    n, Hq, Hkv, D, L = W.P1_PROMPT, w.Hq, w.Hkv, w.D, w.layers
    A, B = W.shared_prompts(2)
    nblk = W.blocks_for(n)
    pc = kvc.PrefixCache(2 * nblk)
    ba = pc.allocate(nblk)
    pc.commit(A, ba)
    t0 = time.perf_counter()
    reps = 200
    for _ in range(reps):
        m = pc.match(B)
        pc.release(m)
    match_us = (time.perf_counter() - t0) / reps * 1e6
    m = pc.match(B)
    start = 16 * len(m)
    fresh = pc.allocate(nblk - len(m))
    caches = [kvc.PagedKVCache.allocate(2 * nblk, Hkv, D, torch.bfloat16, device=dev)
              for _ in range(L)]
    for c in caches:
        c.k_cache.normal_(0, 0.5)
        c.v_cache.normal_(0, 0.5)
    q = torch.empty(n, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    k = torch.empty(n, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    bt_cold = torch.tensor([ba], dtype=torch.int32, device=dev)
    bt_warm = torch.tensor([m + fresh], dtype=torch.int32, device=dev)
    cu_cold = torch.tensor([0, n], dtype=torch.int32, device=dev)
    cu_warm = torch.tensor([0, n - start], dtype=torch.int32, device=dev)
    p_cold = torch.zeros(1, dtype=torch.int32, device=dev)
    p_warm = torch.full((1,), start, dtype=torch.int32, device=dev)

    def cold(i):
        for c in caches:
            kvc.chunked_prefill_attention(c, q, k, v, cu_cold, p_cold, bt_cold, n, out=out)

    ws = torch.empty(max(1, kvc.prefill_workspace_bytes(1, n, n, n, Hq, Hkv, D)),
                     dtype=torch.uint8, device=dev)

    def cold_split(i):
        for c in caches:
            kvc.chunked_prefill_attention(c, q, k, v, cu_cold, p_cold, bt_cold, n, out=out,
                                          max_context_len=n, workspace=ws)

    def warm(i):
        for c in caches:
            kvc.chunked_prefill_attention(c, q[start:], k[start:], v[start:], cu_warm, p_warm,
                                          bt_warm, n - start, out=out[start:],
                                          max_context_len=n, workspace=ws)

    def warm_unsplit(i):
        for c in caches:
            kvc.chunked_prefill_attention(c, q[start:], k[start:], v[start:], cu_warm, p_warm,
                                          bt_warm, n - start, out=out[start:])

    ms_cold_plain = _timed(cold, args.steps, args.warmup)
    ms_cold = min(ms_cold_plain, _timed(cold_split, args.steps, args.warmup))
    ms_warm = _timed(warm, args.steps, args.warmup)
    ms_warm_unsplit = _timed(warm_unsplit, args.steps, args.warmup)
    pairs_cold = Hq * n * (n + 1) // 2
    pairs_warm = Hq * ((n - start) * start + (n - start) * (n - start + 1) // 2)
    res = _base_line(args, "prefix-cached prefill attention time, 2,000-token prompt with 1,800 "
                     "tokens cached, 32 layers (warm)", round(ms_warm, 4), "ms", ms_warm, "bf16",
                     {"workload": "one 2,000-token prompt, first 1,800 tokens shared with a cached "
                                  "prompt, GQA 32/8, head_dim 128, bf16, 32 layers",
                      "prompt": n, "shared": W.P1_SHARED, "matched_blocks": len(m),
                      "prefill_start": start, "layers": L},
                     {"bound": "mfma", "kernel": "chunk_append_kernel + prefill_attention_kernel",
                      "achieved": round(pairs_warm * 4 * D * L / (ms_warm * 1e-3) / 1e12, 1),
                      "peak": 2500.0, "unit": "TFLOP/s",
                      "frac": round(pairs_warm * 4 * D * L / (ms_warm * 1e-3) / 2.5e15, 4),
                      "traffic": None, "avg_us": round(ms_warm * 1e3 / L, 2)})
    res["higher_is_better"] = False
    res["cold_ms"] = round(ms_cold, 4)
    res["cold_ms_without_key_split"] = round(ms_cold_plain, 4)
    res["warm_ms_without_key_split"] = round(ms_warm_unsplit, 4)
    res["cold_tflops"] = round(pairs_cold * 4 * D * L / (ms_cold * 1e-3) / 1e12, 1)
    res["speedup_cold_over_warm"] = round(ms_cold / ms_warm, 2)
    res["host_match_us"] = round(match_us, 1)
    print(json.dumps(res), flush=True)


# the aiwithghost page's simulated queue table (Node on one CPU thread, a tiny
# random-weight model): context for the shape of the results, not a target
PAGE_QUEUE_TABLE = {
    "one at a time, no cache": (452.2, 851.5, 892.3, 64),
    "one at a time, KV cache": (23.9, 45.1, 47.3, 1203),
    "static batches of 16, cache": (21.2, 40.5, 42.8, 1331),
    "continuous batching, 16 slots": (13.8, 26.4, 27.8, 2044),
}


def bench_queue_replay(args):
    """The lab's queue replay on MI355X: 1,000 requests at t = 0 (prompts 8-32,
    answers 16-96 tokens), 16 slots. Step times of the attention path (32
    layers of GQA 32/8/128 bf16 attention: the fused append + decode launch for
    decode rows, the chunked-prefill launch for prompts) are measured over a
    grid of batch rows x lengths, each grid point one HIP graph of the 32
    layers' launches replayed between two events; the native scheduler plans
    every policy and the replay sums interpolated shares, as the lab does.
    Then the leading steps of each continuous plan are run for real (each step
    captured as a graph of its own descriptors) and their measured time is set
    against the estimate for the same steps."""
    import torch

    import kv_cache_decode_append_amd as kvc
    import workloads as W
    from kv_cache_decode_append_amd import replay as R

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.P1
    Hq, Hkv, D, L = w.Hq, w.Hkv, w.D, w.layers
    slots = W.QUEUE_SLOTS
    prompts, answers = W.queue_requests()
    max_blocks = W.blocks_for(max(p + a - 1 for p, a in zip(prompts, answers)))
    nb = slots * max_blocks
    caches = [kvc.PagedKVCache.allocate(nb, Hkv, D, torch.bfloat16, device=dev) for _ in range(L)]
    for c in caches:
        c.k_cache.normal_(0, 0.5)
        c.v_cache.normal_(0, 0.5)
    max_rows = slots * 128
    q = torch.empty(max_rows, Hq, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    kv = torch.empty(max_rows, Hkv, D, dtype=torch.bfloat16, device=dev).normal_(0, 0.5)
    out = torch.empty_like(q)
    scale = 1.0 / D ** 0.5
    reps = max(5, args.steps // 5)

    def graph_ms(launch, reps):
        launch()                      # eager once (also checks the arguments)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launch()
        g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            g.replay()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def decode_launch(n, bt, ctx, max_ctx):
        def run():
            for c in caches:
                kvc.decode_append_attention(c, q[:n], kv[:n], kv[:n], bt, ctx, max_ctx, scale,
                                            out=out[:n])
        return run

    def prefill_launch(total, cu, pre, bt, max_chunk):
        def run():
            for c in caches:
                kvc.chunked_prefill_attention(c, q[:total], kv[:total], kv[:total], cu, pre, bt,
                                              max_chunk, scale, out=out[:total])
        return run

    mws = torch.zeros(kvc.mixed_workspace_bytes(slots, 0, Hq, Hkv, D), dtype=torch.uint8,
                      device=dev)
    out2 = torch.empty_like(out)

    def one_launch(st, dec, pf):
        n, total = len(st.decode_ids), st.prefill_total_tokens
        args = {}
        if n:
            args.update(q_decode=q[:n], k_new=kv[:n], v_new=kv[:n], decode_block_table=dec[0],
                        decode_context_lens=dec[1], decode_max_context=st.decode_max_context,
                        out_decode=out[:n])
        if total:
            args.update(q_prefill=q[:total], k_prefill=kv[:total], v_prefill=kv[:total],
                        cu_chunk_lens=pf[1], prefix_lens=pf[2], prefill_block_table=pf[0],
                        prefill_max_chunk=st.prefill_max_chunk, out_prefill=out2[:total])

        def run():
            for c in caches:
                kvc.mixed_step_attention(c, Hq, softmax_scale=scale, workspace=mws, **args)
        return run

    # 1. the grid
    rows = [1, 2, 4, 8, 16]
    lengths = [8, 16, 24, 32, 48, 64, 96, 128]
    grid_bt = torch.arange(nb, dtype=torch.int32, device=dev).reshape(slots, max_blocks)
    dec_ms = [[0.0] * len(lengths) for _ in rows]
    pf_ms = [[0.0] * len(lengths) for _ in rows]
    t0 = time.perf_counter()
    for i, n in enumerate(rows):
        for j, ln in enumerate(lengths):
            ctx = torch.full((n,), ln, dtype=torch.int32, device=dev)
            dec_ms[i][j] = graph_ms(decode_launch(n, grid_bt[:n], ctx, ln), reps)
            cu = torch.arange(0, (n + 1) * ln, ln, dtype=torch.int32, device=dev)
            pre = torch.zeros(n, dtype=torch.int32, device=dev)
            pf_ms[i][j] = graph_ms(prefill_launch(n * ln, cu, pre, grid_bt[:n], ln), reps)
        print(f"[queue-replay] grid rows={n} done ({time.perf_counter() - t0:.1f} s)",
              file=sys.stderr, flush=True)
    times = R.StepTimes(rows, lengths, dec_ms, pf_ms)

    # 2. plans and the replay estimate
    answer_tokens = int(sum(answers))
    table, plans = {}, {}
    for pol in R.queue_policies(slots):
        steps = R.plan(pol, prompts, answers)
        costs = [R.step_cost_ms(st, times, pol.recompute) for st in steps]
        res = R.replay(steps, costs, len(prompts))
        summ = R.summarize(res, answer_tokens)
        summ = {k: round(v, 4) for k, v in summ.items()}
        summ["steps"] = len(steps)
        table[pol.name] = summ
        plans[pol.name] = (steps, costs)
    print(f"[queue-replay] replay done ({time.perf_counter() - t0:.1f} s)", file=sys.stderr,
          flush=True)

    # 3. the leading steps of the continuous plans, run for real
    direct = {}
    for name in (f"continuous batching, {slots} slots",
                 f"continuous batching, {slots} slots, decode first"):
        steps, costs = plans[name]
        k = min(args.direct_steps, len(steps))
        real = real_one = 0.0
        for st in steps[:k]:
            parts = []
            dec = pf = None
            if len(st.decode_ids):
                n = len(st.decode_ids)
                dec = (torch.from_numpy(st.decode_block_table).to(dev),
                       torch.from_numpy(st.decode_context_lens).to(dev))
                parts.append(decode_launch(n, dec[0], dec[1], st.decode_max_context))
            if len(st.prefill_ids):
                pf = (torch.from_numpy(st.prefill_block_table).to(dev),
                      torch.from_numpy(st.prefill_cu_chunk_lens).to(dev),
                      torch.from_numpy(st.prefill_prefix_lens).to(dev))
                parts.append(prefill_launch(st.prefill_total_tokens, pf[1], pf[2], pf[0],
                                            st.prefill_max_chunk))
            real += graph_ms(lambda: [f() for f in parts], 3)
            real_one += graph_ms(one_launch(st, dec, pf), 3)
        est = float(sum(costs[:k]))
        direct[name] = {"steps": k, "measured_ms": round(real, 3), "estimated_ms": round(est, 3),
                        "measured_over_estimated": round(real / est, 4),
                        "measured_one_launch_ms": round(real_one, 3),
                        "one_launch_speedup": round(real / real_one, 4)}
        print(f"[queue-replay] direct {name}: {k} steps ({time.perf_counter() - t0:.1f} s)",
              file=sys.stderr, flush=True)

    head = table[f"continuous batching, {slots} slots"]
    res = _base_line(args, "queue replay answer tokens/s, continuous batching with 16 slots, "
                     "1,000 requests at t = 0 (attention path, 32 layers, measured step times)",
                     round(head["tokens_per_s"], 1), "tokens/s",
                     head["all_done_s"] * 1e3 / head["steps"], "bf16",
                     {"workload": "1,000 requests at t = 0, prompts 8-32 tokens, answers 16-96 "
                                  "tokens (uniform), 16 slots, GQA 32/8, head_dim 128, bf16, "
                                  "32 layers of attention per step",
                      "requests": len(prompts), "answer_tokens": answer_tokens, "slots": slots,
                      "prefill_token_budget": 2048, "layers": L},
                     None)
    res["steps"] = head["steps"]
    res["warmup"] = 1
    res["queue_table"] = table
    res["page_queue_table"] = {k: dict(zip(("median_ttft_s", "p95_ttft_s", "all_done_s",
                                            "tokens_per_s"), v))
                               for k, v in PAGE_QUEUE_TABLE.items()}
    res["step_time_grid_ms"] = {"rows": rows, "lengths": lengths, "decode": dec_ms,
                                "prefill": pf_ms}
    res["direct_check"] = direct
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
