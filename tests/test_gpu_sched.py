"""GPU parity for the serving loop: the native scheduler plans each step and
builds its batch descriptors (include/kvc_sched.h), and the kernels run them:
kvc_decode_append_attention for the decode rows, then
kvc_chunked_prefill_attention(_split) for the prompt chunks, on one stream.
Every output row is compared with the oracle's attention over that request's
positions so far. Block ids are reused as requests leave, and the pool starts
as NaN, so a descriptor that points at a stale or unwritten block shows up.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import FILL, assert_close, oracle_values, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvc():
    import kv_cache_decode_append_amd as m
    return m


def run_queue(kvc, policy, prompts, answers, slots, budget, dtype, Hq, Hkv, D, split, wid,
              one_launch=False):
    dev = torch.device("cuda")
    n = len(prompts)
    w = W.small_workload(f"sched-{wid}", wid, B=n, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, sigma=0.5)
    vals = [W.sequence_values(w, r, p + a, p + a) for r, (p, a) in enumerate(zip(prompts, answers))]
    max_blocks = W.blocks_for(max(p + a - 1 for p, a in zip(prompts, answers)))
    nb = slots * max_blocks
    sched = kvc.Scheduler(policy, slots, budget, nb, max_blocks)
    for p, a in zip(prompts, answers):
        sched.submit(p, a)
    cache = kvc.PagedKVCache.allocate(nb, Hkv, D, W_T[dtype], device=dev, fill_bits=FILL)
    scale = 1.0 / D ** 0.5
    ov = [tuple(oracle_values(x, dtype) for x in v) for v in vals]
    worst, n_steps, rows = 0.0, 0, 0
    ws = torch.zeros(kvc.mixed_workspace_bytes(slots, 0, Hq, Hkv, D), dtype=torch.uint8,
                     device=dev) if one_launch else None
    while (st := sched.next_step()) is not None:
        n_steps += 1
        if one_launch:
            worst = max(worst, _one_launch_step(kvc, cache, st, vals, ov, dtype, Hq, scale, ws))
            rows += len(st.decode_ids) + int(st.prefill_cu_chunk_lens[-1])
            continue
        if len(st.decode_ids):
            ids, ctx = st.decode_ids, st.decode_context_lens
            q = np.stack([vals[r][2][c - 1] for r, c in zip(ids, ctx)])
            k = np.stack([vals[r][0][c - 1] for r, c in zip(ids, ctx)])
            v = np.stack([vals[r][1][c - 1] for r, c in zip(ids, ctx)])
            out = kvc.decode_append_attention(
                cache, to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                torch.from_numpy(st.decode_block_table).to(dev),
                torch.from_numpy(ctx).to(dev), st.decode_max_context, scale)
            got = out.float().cpu().numpy()
            for i, (r, c) in enumerate(zip(ids, ctx)):
                kk, vv, qq = ov[r]
                ref = OA.attend_row(qq[c - 1], kk[:c], vv[:c], scale)
                worst = max(worst, assert_close(got[i], ref, dtype, f"decode r{r} ctx {c}"))
            rows += len(ids)
        if len(st.prefill_ids):
            ids, pre, cu = st.prefill_ids, st.prefill_prefix_lens, st.prefill_cu_chunk_lens
            spans = [(int(r), int(s0), int(s0 + cu[i + 1] - cu[i])) for i, (r, s0) in
                     enumerate(zip(ids, pre))]
            q = np.concatenate([vals[r][2][s0:e] for r, s0, e in spans])
            k = np.concatenate([vals[r][0][s0:e] for r, s0, e in spans])
            v = np.concatenate([vals[r][1][s0:e] for r, s0, e in spans])
            out = kvc.chunked_prefill_attention(
                cache, to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                torch.from_numpy(cu).to(dev), torch.from_numpy(pre).to(dev),
                torch.from_numpy(st.prefill_block_table).to(dev), st.prefill_max_chunk, scale,
                max_context_len=st.prefill_max_context if split else None)
            got = out.float().cpu().numpy()
            for i, (r, s0, e) in enumerate(spans):
                kk, vv, qq = ov[r]
                for t in range(s0, e):
                    ref = OA.attend_row(qq[t], kk[:t + 1], vv[:t + 1], scale)
                    worst = max(worst, assert_close(got[cu[i] + t - s0], ref, dtype,
                                                    f"prefill r{r} pos {t}"))
            rows += int(cu[-1])
    torch.cuda.synchronize()
    assert int(cache.err_flag.item()) == 0
    assert sched.unfinished() == 0
    return n_steps, rows, worst


W_T = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _one_launch_step(kvc, cache, st, vals, ov, dtype, Hq, scale, ws):
    """The whole step as one kvc_mixed_step_attention call."""
    dev = torch.device("cuda")
    args = {}
    if len(st.decode_ids):
        ids, ctx = st.decode_ids, st.decode_context_lens
        args.update(
            q_decode=to_device(np.stack([vals[r][2][c - 1] for r, c in zip(ids, ctx)]), dtype),
            k_new=to_device(np.stack([vals[r][0][c - 1] for r, c in zip(ids, ctx)]), dtype),
            v_new=to_device(np.stack([vals[r][1][c - 1] for r, c in zip(ids, ctx)]), dtype),
            decode_block_table=torch.from_numpy(st.decode_block_table).to(dev),
            decode_context_lens=torch.from_numpy(ctx).to(dev),
            decode_max_context=st.decode_max_context)
    spans = []
    if len(st.prefill_ids):
        ids, pre, cu = st.prefill_ids, st.prefill_prefix_lens, st.prefill_cu_chunk_lens
        spans = [(int(r), int(s0), int(s0 + cu[i + 1] - cu[i])) for i, (r, s0) in
                 enumerate(zip(ids, pre))]
        args.update(
            q_prefill=to_device(np.concatenate([vals[r][2][s0:e] for r, s0, e in spans]), dtype),
            k_prefill=to_device(np.concatenate([vals[r][0][s0:e] for r, s0, e in spans]), dtype),
            v_prefill=to_device(np.concatenate([vals[r][1][s0:e] for r, s0, e in spans]), dtype),
            cu_chunk_lens=torch.from_numpy(cu).to(dev), prefix_lens=torch.from_numpy(pre).to(dev),
            prefill_block_table=torch.from_numpy(st.prefill_block_table).to(dev),
            prefill_max_chunk=st.prefill_max_chunk)
    out_dec, out_pf = kvc.mixed_step_attention(cache, Hq, softmax_scale=scale, workspace=ws, **args)
    worst = 0.0
    if out_dec is not None:
        got = out_dec.float().cpu().numpy()
        for i, (r, c) in enumerate(zip(st.decode_ids, st.decode_context_lens)):
            kk, vv, qq = ov[r]
            ref = OA.attend_row(qq[c - 1], kk[:c], vv[:c], scale)
            worst = max(worst, assert_close(got[i], ref, dtype, f"one-launch decode r{r} ctx {c}"))
    if out_pf is not None:
        got = out_pf.float().cpu().numpy()
        cu = st.prefill_cu_chunk_lens
        for i, (r, s0, e) in enumerate(spans):
            kk, vv, qq = ov[r]
            for t in range(s0, e):
                ref = OA.attend_row(qq[t], kk[:t + 1], vv[:t + 1], scale)
                worst = max(worst, assert_close(got[cu[i] + t - s0], ref, dtype,
                                                f"one-launch prefill r{r} pos {t}"))
    assert int(ws[:256].count_nonzero().item()) == 0
    return worst


@pytest.mark.parametrize("policy_name,dtype,split", [
    ("decode_first", "bf16", False), ("decode_first", "bf16", True),
    ("prefill_first", "bf16", False), ("static", "bf16", False), ("decode_first", "fp32", False)])
def test_serving_loop_matches_oracle(kvc, policy_name, dtype, split):
    policy = {"decode_first": kvc.SCHED_DECODE_FIRST, "prefill_first": kvc.SCHED_PREFILL_FIRST,
              "static": kvc.SCHED_STATIC}[policy_name]
    rng = np.random.default_rng(31)
    n = 14
    prompts = rng.integers(1, 150, n).tolist()
    answers = rng.integers(1, 12, n).tolist()
    say(f"serving loop {policy_name} {dtype} split={split}: {n} requests, 4 slots, budget 40")
    steps, rows, worst = run_queue(kvc, policy, prompts, answers, 4, 40, dtype, 8, 2, 128, split,
                                   311)
    say(f"  {steps} steps, {rows} rows, max abs err {worst:.2e}")


def test_serving_loop_long_prompt_chunks(kvc):
    """A 700-token prompt prefilled in budget-sized chunks over its own cached
    prefix while short requests decode (GQA 32/8/128, bf16)."""
    prompts, answers = [9, 700, 20, 33, 5], [30, 4, 25, 6, 9]
    say("serving loop with a 700-token prompt, budget 256")
    steps, rows, worst = run_queue(kvc, kvc.SCHED_DECODE_FIRST, prompts, answers, 3, 256, "bf16",
                                   32, 8, 128, True, 312)
    say(f"  {steps} steps, {rows} rows, max abs err {worst:.2e}")


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("fp32", 8, 2, 32)])
def test_serving_loop_one_launch_per_step(kvc, dtype, Hq, Hkv, D):
    """Decode-first steps from the step builder, each run as ONE mixed launch
    (kvc_mixed_step_attention) over the builder's own descriptors."""
    rng = np.random.default_rng(33)
    n = 12
    prompts = rng.integers(1, 300, n).tolist()
    answers = rng.integers(1, 10, n).tolist()
    say(f"serving loop, one launch per step, {dtype} {Hq}/{Hkv}/{D}: {n} requests, 4 slots, "
        f"budget 96")
    steps, rows, worst = run_queue(kvc, kvc.SCHED_DECODE_FIRST, prompts, answers, 4, 96, dtype,
                                   Hq, Hkv, D, False, 313, one_launch=True)
    say(f"  {steps} steps, {rows} rows, max abs err {worst:.2e}")
