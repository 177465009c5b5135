"""fp64 CPU oracle for paged attention — TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product. Only the test suite, the smoke
check and the bench's CPU-baseline leg may import or run it; the library's own
path never does (it fails loudly when its HIP build is missing).

It is a plain, slow, obviously correct restatement of what the pages define:
  * PagedAttention changes where K and V live, not what attention computes:
    K/V are gathered through a per-sequence block table from fixed-size blocks
    ("Module 4 · Batching, Scheduling, and Paging", section "PagedAttention").
  * Each request's query attends only over that request's own tokens with
    softmax(Q K^T / sqrt(d_k)) V (worksonmygpu.com continuous-batching post,
    section "Selective batching: why this isn't free for attention").
  * The cache grows token by token ("Paging the KV Cache", section "The waste
    hiding inside memory"); shared blocks are copied on the first divergent
    write ("Module 4", section "Block sharing").

Every function is pinned in tests/test_oracle_*.py against facts other than
itself (closed forms, hand-derived examples under tests/golden/, a library
attention routine on contiguous inputs, invariants, and the independent
pure-Python brute force in ``oracle.brute``). No function here is unpinned.
"""
from .paged_attention import (append, attend, attend_partitioned, check_slots, copy_blocks,
                              decode, decode_elements, decode_moments, gather, merge_partials,
                              pool_views, prefill, prefill_moments, softmax_moments,
                              swap_blocks)

__all__ = ["append", "attend", "attend_partitioned", "check_slots", "copy_blocks", "decode",
           "decode_elements", "decode_moments", "gather", "merge_partials", "pool_views",
           "prefill", "prefill_moments", "softmax_moments", "swap_blocks"]
