"""One continuous-batching step's attention, run by whichever launch route is
faster on this device for steps of its size.

A step holds decode rows (each writes its newest K/V and attends over its
whole context) and prompt chunks (each writes its K/V and attends causally over
its cached prefix): the batch a continuous-batching server rebuilds every
step (aiwithghost.com "KV cache and continuous batching: 1,000 people ask AI",
section "How does continuous batching share the server?"; gouthm.com "The KV
cache is not your bottleneck", section "The fix that mattered"). The library
runs such a step two ways:

  * separate launches: decode_append_attention for the decode rows, then
    chunked_prefill_attention for the chunks, on one stream;
  * one launch: mixed_step_attention, a persistent kernel that takes both
    kinds of items from one device queue.

Both write the same cache bytes and the same prefill rows, bit for bit; the
decode rows differ in summation order only (the one-launch kernel walks a
row's blocks with the 8 waves of one workgroup instead of splitting long rows
over workgroups), so both are within the same tolerance of exact attention.

The rule StepRunner applies (route="auto"):

  * a step with only decode rows or only chunks takes its own call: the
    one-launch kernel would run the same items with fewer blocks in flight
    per decode wave (its prefill items set its register budget) and the
    queue's set-up on top;
  * a step with both kinds is put in a size class (the power of two at or
    above its number of decode rows, its longest decode context and its
    prompt tokens). Its first steps alternate the routes and are timed (the
    stream is synchronised around them): on each route the first step warms
    up (first use of a kernel, caches) and is not counted, the next `trials`
    are. From then on the class takes the one launch only if its median time
    beat the separate launches' median by more than `margin`, and the
    separate launches otherwise. A configuration the one-launch kernel does not
    support (KVC_ERR_UNSUPPORTED) takes the separate launches.

route="separate" or "one_launch" fixes the route instead. The choice for a
class is kept for the runner's lifetime (`decisions`), so the route of a step
of a decided class never changes.
"""
from __future__ import annotations

import statistics

import torch

from . import _lib

SEPARATE, ONE_LAUNCH = "separate", "one_launch"
KVC_ERR_UNSUPPORTED = -4


def _size_class(n: int) -> int:
    """The power of two at or above n (0 for n <= 0)."""
    return 0 if n <= 0 else 1 << (int(n) - 1).bit_length()


def _event_timer(fn):
    """Runs fn() between two synchronisations and returns (result, ms)."""
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    res = fn()
    ev1.record()
    torch.cuda.synchronize()
    return res, ev0.elapsed_time(ev1)


class StepRunner:
    """Runs steps over one cache (one layer's pools, or several layers' pools
    of the same shape in turn) by the route described in the module docstring.

    decode = dict(q, k_new, v_new, block_table, context_lens, max_context)
    prefill = dict(q, k, v, cu_chunk_lens, prefix_lens, block_table, max_chunk)
    (with the shapes decode_append_attention and chunked_prefill_attention
    take); either may be None or empty. run() returns (out_decode,
    out_prefill), None for an empty part."""

    def __init__(self, Hq: int, softmax_scale: float | None = None, route: str = "auto",
                 trials: int = 3, margin: float = 0.02, timer=None):
        if route not in ("auto", SEPARATE, ONE_LAUNCH):
            raise ValueError(f"unknown route {route!r}")
        if trials < 1 or not 0.0 <= margin < 1.0:
            raise ValueError("trials >= 1 and 0 <= margin < 1")
        self.Hq, self.scale, self.route = Hq, softmax_scale, route
        self.trials, self.margin = trials, margin
        self.timer = timer or _event_timer
        self.decisions: dict[tuple, str] = {}
        self.samples: dict[tuple, dict[str, list]] = {}
        self._mws = None            # the one-launch workspace (zeroed header), grown on demand

    # ---------------------------------------------------------------- the rule
    @staticmethod
    def size_class(n_decode: int, decode_max_context: int, prefill_tokens: int) -> tuple:
        return (_size_class(n_decode), _size_class(decode_max_context),
                _size_class(prefill_tokens))

    def pick(self, n_decode: int, decode_max_context: int, prefill_tokens: int):
        """(route, class key or None): the route for a step of these sizes, and
        the key its time is recorded under while its class is being timed."""
        if self.route != "auto":
            return self.route, None
        if n_decode <= 0 or prefill_tokens <= 0:
            return SEPARATE, None
        key = self.size_class(n_decode, decode_max_context, prefill_tokens)
        if key in self.decisions:
            return self.decisions[key], None
        s = self.samples.setdefault(key, {SEPARATE: [], ONE_LAUNCH: []})
        return (SEPARATE if len(s[SEPARATE]) <= len(s[ONE_LAUNCH]) else ONE_LAUNCH), key

    def record(self, key: tuple, route: str, ms: float) -> None:
        """Adds a timed step of class `key` (the first on each route is the
        warm-up); decides the class once both routes have `trials` counted
        samples."""
        s = self.samples[key]
        s[route].append(float(ms))
        counted = {r: s[r][1:] for r in (SEPARATE, ONE_LAUNCH)}
        if min(len(v) for v in counted.values()) >= self.trials:
            sep, one = statistics.median(counted[SEPARATE]), statistics.median(counted[ONE_LAUNCH])
            self.decisions[key] = ONE_LAUNCH if one < sep * (1.0 - self.margin) else SEPARATE

    # ---------------------------------------------------------------- running
    def run(self, cache, decode: dict | None = None, prefill: dict | None = None):
        n_dec = 0 if decode is None else int(decode["q"].shape[0])
        n_pf = 0 if prefill is None else int(prefill["q"].shape[0])
        dec_max = int(decode["max_context"]) if n_dec else 0
        route, key = self.pick(n_dec, dec_max, n_pf)
        if key is None:
            return self._run(route, cache, decode if n_dec else None, prefill if n_pf else None)
        try:
            res, ms = self.timer(lambda: self._run(route, cache, decode, prefill))
        except _lib.KvcError as e:
            if route != ONE_LAUNCH or e.status != KVC_ERR_UNSUPPORTED:
                raise
            self.decisions[key] = SEPARATE        # validated before any launch: nothing ran
            return self._run(SEPARATE, cache, decode, prefill)
        self.record(key, route, ms)
        return res

    def _run(self, route: str, cache, decode, prefill):
        if route == ONE_LAUNCH and decode is not None and prefill is not None:
            return self._one_launch(cache, decode, prefill)
        out_dec = out_pf = None
        if decode is not None:
            out_dec = _lib.decode_append_attention(
                cache, decode["q"], decode["k_new"], decode["v_new"], decode["block_table"],
                decode["context_lens"], int(decode["max_context"]), self.scale)
        if prefill is not None:
            out_pf = _lib.chunked_prefill_attention(
                cache, prefill["q"], prefill["k"], prefill["v"], prefill["cu_chunk_lens"],
                prefill["prefix_lens"], prefill["block_table"], int(prefill["max_chunk"]),
                self.scale)
        return out_dec, out_pf

    def _one_launch(self, cache, decode, prefill):
        n_dec = int(decode["q"].shape[0])
        need = max(256, _lib.mixed_workspace_bytes(n_dec, int(decode["max_context"]), self.Hq,
                                                   cache.num_kv_heads, cache.head_dim))
        dev = cache.k_cache.device
        if self._mws is None or self._mws.numel() < need or self._mws.device != dev:
            self._mws = torch.zeros(need, dtype=torch.uint8, device=dev)
        return _lib.mixed_step_attention(
            cache, self.Hq, q_decode=decode["q"], k_new=decode["k_new"], v_new=decode["v_new"],
            decode_block_table=decode["block_table"], decode_context_lens=decode["context_lens"],
            decode_max_context=int(decode["max_context"]), q_prefill=prefill["q"],
            k_prefill=prefill["k"], v_prefill=prefill["v"],
            cu_chunk_lens=prefill["cu_chunk_lens"], prefix_lens=prefill["prefix_lens"],
            prefill_block_table=prefill["block_table"], prefill_max_chunk=int(prefill["max_chunk"]),
            softmax_scale=self.scale, workspace=self._mws)
