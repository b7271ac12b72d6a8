"""CPU oracle for the paged KV-cache decode/append path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product (the
HIP library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product.

Everything here is plain, slow and meant to be read against the pages:

* ``attention``: scaled dot-product attention of one query row over a prefix of
  cached keys/values, the naive recompute-everything generation loop, the
  cached loop, decode rows and prefill-chunk rows (fp64 arithmetic).
* ``paged``: block-table bookkeeping, slot numbers, the expected cache pool
  after writes, gathering a sequence back out of the pool.
* ``bf16``: round-to-nearest-even fp32 -> bfloat16 by bit arithmetic.
* ``sizes``: KV bytes per token and the capacity arithmetic.
* ``prefix``: prefix caching, i.e. whole-block matching of a prompt's opening
  tokens against cached blocks, with reference counts and block reuse.
* ``quant``: fp8 (E4M3) quantisation of KV rows with one scale per token and
  kv head.
* ``sched``: iteration-level scheduling of a request queue (continuous
  batching under decode-first or prefill-first steps, static batching).

Every function is pinned by a CPU test (``tests/test_oracle_*.py``) against
values the pages print, closed forms, special cases, library routines or
brute force; see each function's docstring for its pin.
"""
from . import attention, bf16, paged, prefix, quant, sched, sizes  # noqa: F401
