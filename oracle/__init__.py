"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition of what the
HIP library computes.  It exists to check that library and for nothing
else: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``paged_kv_cache_253_amd``) never imports it, and it never imports the
product path; the two share no code, headers, tables or constants.  The
only shared module is the seeded input generator (``workloads``), which
holds none of the method's arithmetic.

Sources (the three web pages on paged KV caches):

* "AI Inference Serving at Scale: vLLM, TensorRT-LLM, PagedAttention, and
  KV-Cache Optimization" -- section 3 (physical block pool, block table,
  on-demand allocation, copy-on-write sharing), section 2 (dot-product
  attention against every cached token), section 6 (FP8 KV cache, GQA),
  FAQ ("paged attention is identical to un-paged attention").
* "How LLM Inference Engines Work: KV Caches, PagedAttention, and
  Continuous Batching" -- section "PagedAttention: Virtual Memory for KV
  Caches" (pages of 16 or 32 tokens, the kernel gathers K and V from
  non-adjacent memory).
* "vLLM & High-Throughput Serving" -- section 1 (contiguous K/V layout,
  token t attends to the cached tokens before it), section 2 (block-table
  equation: logical block i = floor(t / B), offset j = t mod B).

Floating point is fp64 throughout: bf16 and e4m3 values are exact in
fp64, so the only rounding is the fp64 arithmetic of the textbook
formulas.  Every function states which passage it follows.

Parity status of each function (what pins it is listed in the tests):

* ``codecs.bf16_bits_to_f64``, ``codecs.e4m3_to_f64``,
  ``codecs.e4m3_encode`` -- pinned (library dtype tables, format limits).
* ``paged.write_tokens``, ``paged.gather`` -- pinned (hand-worked golden
  example, brute-force scatter/gather round trip, untouched-slot checks).
* ``paged.attention``, ``paged.decode`` -- pinned by invariants and closed
  forms (permutation, paged == unpaged, shared == copied prefix, L = 1,
  L = 2, identical keys, saturation, library SDPA, pure-Python brute
  force).  No page prints attention output values, so nothing external
  fixes the output digits beyond those.
* ``paged.partial``, ``paged.merge`` -- pinned (merge of any split equals
  the unsplit result; single partition is the identity).
"""

from . import codecs, paged  # noqa: F401

__all__ = ["codecs", "paged"]
