"""CPU oracle for chunked-prefill / prefix-cached paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constant tables); the only common
dependency is the ``synth`` input generator, which holds no method arithmetic.

Everything is written as the plain definition, in float64, from these pages:

* "Prefill Processing" (Neuron vLLM design page): chunk iterations, cached
  segments of ``kv_segment_size``, partial-segment masking, metadata, block
  allocation.
* "Prefill Optimisation: Prefix Caching, Chunked Prefill, and
  Disaggregation" (tutorial): causal equivalence (section 2), token budget
  (section 2, section 7), pair and FLOP arithmetic (section 4), KV bytes
  (section 6).
* "Chunked Prefill" (blog note): decode-first budget fill with a per-prefill
  chunk cap.
* "vLLM Chunked Prefill 如何改变 KV Cache 管理": incremental block
  allocation (section 2.1), block-aligned budget (section 2.3).

``prefix_cache`` and the prefix-caching part of ``schedule`` follow the
parent-chained block identity (kept exact: a trie of token blocks instead
of a digest), full-block matching and the pool's three buckets
("Prefill Optimisation ...", sections 3 and 7) and the first-chunk-only
lookup ("vLLM Chunked Prefill ...", sections 2.2 and 3.1).

``fp8`` has the E4M3 code of a cache element (per-tensor scale) and its
value, for a cache kept in FP8 ("Prefill Optimisation ...", section 3 names
the element type as part of a cache entry; the format itself is the
standard OCP one).

``rope`` adds rotary position embedding at absolute positions ("Prefill
Optimisation ...", section 2, "Causal equivalence"; "Chunked Prefill",
section "From scratch"), in the standard rotary form, which the pages name
but do not write out.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against printed values, closed forms, a library routine or an invariant.
The one reading without a pin of its own is the GQA head grouping (the pages
never define it); it is fixed to the consecutive grouping that
``torch.nn.functional.scaled_dot_product_attention`` uses and is pinned only
against that library convention.
"""
from . import attention, counters, fp8, prefix_cache, rope, schedule  # noqa: F401
