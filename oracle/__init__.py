"""CPU oracle for the paged-KV decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the benchmark's GPU legs) may import, call or link this
package.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.

It is a plain, slow, obviously-correct implementation of what the paged KV
cache computes, written from three web pages on the subject:

* P1: "Paged Attention" (klaylearn.com glossary)
* P2: "PagedAttention — AI Glossary" (modelrefs.com)
* P3: "What is paged attention in vLLM, and why does it matter?"
  (interview.clozo.ai blog)

Every function names the page and section it follows.  Floating point work
is done in float64; stored bf16 values are widened exactly.  The package
shares no code with the HIP path: it imports only numpy, scipy and the
standard library, and takes every input (including all random numbers) as
arguments.

Modules
-------
allocator   block allocator: free stack, per-block reference counts,
            per-sequence block tables, lazy allocation, fork, copy-on-write
cache_ops   slot-mapped append and whole-block copy (exact bit copies)
attention   paged single-query attention (gather through the block table),
            contiguous-cache attention, scalar brute force
prefill     paged multi-query (prefill / chunked prefill) causal attention,
            a dense masked formulation, scalar brute force
accounting  the pages' memory arithmetic (bytes per token, slab vs block
            utilisation, tail waste, capacity)

Parity status: every function here is pinned by tests under ``tests/``
(``-m "not gpu"``) against values the pages print, closed forms, library
routines or brute force.  No function is "parity unpinned".
"""

from . import accounting, allocator, attention, cache_ops  # noqa: F401
