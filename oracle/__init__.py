"""CPU oracle for paged decode attention - TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct reference for what the GPU library
computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the product path (the C-ABI library and
its Python binding) never does, and the oracle imports nothing from the
product path either. The two share only the seeded input generators in
``workloads/``, which hold none of the method's arithmetic.

Pages cited throughout the oracle:
  [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
  [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
  [KVM] "深入解析 vLLM 的 KV Cache 管理器：从内存碎片到 PagedAttention 的完整技术剖析"
        (zingnex.cn)

Modules:
  attention   - gather through the block table, dense fp64 softmax attention;
                the five-step blockwise softmax and the split-context merge.
  cache_ops   - bitwise K/V append into slots and whole-block copies.
  alloc_model - the block allocator: FIFO free list, reference counts,
                per-sequence block tables, fork, copy-on-write, free.
  sizes       - the closed-form sizes and waste figures the pages print.
  runner      - replays a workload's host operations with the pieces above.

Every function is pinned by tests that check it against what the pages and
the mathematics fix (printed figures, closed forms, invariants, brute force
on tiny inputs, special cases); none is "parity unpinned".
"""
