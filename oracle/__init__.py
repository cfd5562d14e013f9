"""Oracle for paged KV-cache decode: a plain, slow CPU implementation in float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
this package imports nothing from the product path: the two share no code.

What it computes, and the passage each part follows:

* ``block_manager``  - logical->physical block tables, on-demand allocation and
  copy-on-write of refcounted blocks (agentalpha.top Q32 answer parts 2-3;
  data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache"; ohmygp.com "破局思路").
* ``kv_cache``       - the physical pool, the KV write into a slot, and the block copy.
* ``attention``      - decode attention gathered through the block table, the
  partitioned form with a log-sum-exp merge, and causal attention of a chunk of new
  tokens (prefill / chunked prefill) over the same pool.
* ``accounting``     - the memory-waste accounting of the ohmygp.com simulation.
* ``tables``         - flat, 16-bit and two-level block tables and their memory
  (agentalpha.top Q32 follow-up 1).
* ``replay``         - replays a ``synth`` workload through the parts above.

Every function here is pinned by a ``-m "not gpu"`` test against something other
than itself (worked examples from the pages, closed forms, library routines,
brute force on tiny inputs); no function is "parity unpinned".
"""
from . import accounting, attention, block_manager, kv_cache, numerics, replay, tables  # noqa: F401
