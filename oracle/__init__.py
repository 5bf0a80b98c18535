"""Plain CPU oracle for chunked prefill attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links this package; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` do.

It computes, in float64 with numpy, exactly what the pages define:

* ``attention``: gather pages into contiguous K/V through the block table,
  then causal softmax(Q K^T / sqrt(d)) V with grouped-query heads
  (issue "Metal: paged-KV prefill is 4.43x slower than contiguous KV at 32K",
  TL;DR and "Results": paged and contiguous KV are the same computation, only
  the storage differs).
* the split form: the key axis cut into ranges, one partial per range, merged
  by log-sum-exp (PR "perf: scale prefill attention splits with GPU cores on
  Apple7/8", "What changed" and "Testing": the reduce sums S partials).
* ``rules``: the page's split-count rule and piece-size rule, transcribed from
  the same PR ("What changed" and the explanatory note below "Testing").
* ``kv_append``: the chunk's K/V rows written into their pages through the
  block table (the issue's publishing of completed KV pages, after its
  "Expected vs actual" table).
* ``quant``: 8-bit K/V pages (q8_0's 32-value blocks with an fp16 scale),
  dequantized in the gather, and the quantizing append (the 8-bit KV cache
  types of the KVarN report and of the speculative-decoding page).
* ``varlen_paged_attention``: a packed batch of sequences, each with its own
  history, rows and block table over one shared pool (the serving setting of
  the issue's problem statement: continuous batching, prefix caching).

Every function is pinned by ``tests/test_oracle_pins.py`` against brute force,
closed forms, torch's CPU attention with an explicit mask, invariants, and the
values the PR prints for its split and piece tables.
"""

from .attention import (  # noqa: F401
    decode_f16,
    decode_bf16,
    gather_pages,
    causal_attention,
    paged_causal_attention,
    page_aligned_split_ranges,
    split_partials,
    merge_partials,
    split_causal_attention,
    causal_attention_rows,
)
from .rules import page_split_rule, page_piece_rows  # noqa: F401
from .cache import kv_append  # noqa: F401
from .varlen import varlen_paged_attention  # noqa: F401
from .quant import (  # noqa: F401
    quantize_q8,
    dequantize_q8,
    decode_scales,
    paged_q8_attention,
    kv_append_q8,
)
