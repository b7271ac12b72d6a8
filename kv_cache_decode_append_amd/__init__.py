"""Paged KV-cache append, GQA decode attention and chunked-prefill attention on
AMD MI355X (gfx950): HIP kernels behind the C ABI in include/kvc.h, with this
thin binding on top, and a host-side prefix-caching block manager
(include/kvc_prefix.h), and an iteration-level scheduler that builds each
step's batch descriptors (include/kvc_sched.h), and a step runner that picks the faster launch
route for a step of decode rows and prompt chunks (step.py). Importing the package loads libkvc.so and raises if it is
missing; there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE,
    DEVERR_BLOCK_ID,
    DEVERR_CONTEXT,
    DEVERR_QUEUE,
    DEVERR_SLOT,
    KVC_BF16,
    KVC_F32,
    KVC_FP8,
    LIB,
    LIB_PATH,
    KvcError,
    PagedKVCache,
    PrefixCache,
    SCHED_DECODE_FIRST,
    SCHED_PREFILL_FIRST,
    SCHED_STATIC,
    SchedStep,
    Scheduler,
    chunked_prefill_attention,
    decode_append_attention,
    decode_append_attention_noalloc,
    decode_workspace_bytes,
    kv_append,
    kv_bytes_per_token,
    mixed_step_attention,
    mixed_workspace_bytes,
    paged_decode_attention,
    prefill_workspace_bytes,
    slot_mapping,
    stream_read,
)
from .step import ONE_LAUNCH, SEPARATE, StepRunner  # noqa: F401
