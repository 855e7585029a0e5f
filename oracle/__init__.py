"""Plain, slow, obviously-correct CPU oracle for the paged KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``paged_kv_cache_431_amd``) and imports nothing from it.

Everything is NumPy float64 (the integer parts are plain Python / NumPy int64).
The modules follow the pages that describe the method; citations name the page
and the section on it:

  [UD]  understandingdata.com -- "AI Engineering Visualised: KV cache"
        (sections: intro, "The maths").
  [OT]  optiverse-tech.com blog -- "Paged KV Cache" tutorial, first heading
        "Managing the KV Cache" (sections: "Reproduce Bytes per Token",
        "Worked Example: The 825-Token Request", "Worked Capacity Under a
        12 GiB KV Budget", "Block Tables and Sharing", "Quantized KV",
        "Build the Capacity Calculator", "Deliberately Broken Cases",
        "Answer Key").
  [AF]  aifrontierpost.com -- "KV cache and PagedAttention in serving"
        (sections: "What the KV cache actually is", "PagedAttention: virtual
        memory for GPUs", "The bonus: sharing via copy-on-write").

Modules
  codecs     -- element codecs (bf16 / f16 / f32 / fp8 e4m3) decoded from bits.
  attention  -- paged attention: resolve block tables, textbook softmax; decode
                (one new token) and several new tokens with a causal mask.
  scatter    -- reshape_and_cache: write each new token's K/V into its slot.
  copy       -- copy_blocks: the block copy of copy-on-write.
  allocator  -- block manager: FIFO free list, refcounts, fork, copy-on-write.
  capacity   -- the pages' sizing arithmetic (bytes/token, slots, blocks).

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against values the pages print, closed forms, a
library routine, or brute force; none is "parity unpinned".
"""

from . import allocator, attention, capacity, codecs, copy, scatter  # noqa: F401
