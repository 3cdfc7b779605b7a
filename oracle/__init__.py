"""CPU FP64 oracle for BF16 attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never imports, links or calls it, and it shares no code with the HIP
library: the two meet only in the seeded inputs of the ``workloads`` package.

What it computes, and where the pages define it:

* ``attention``: softmax attention evaluated straight from its definition in
  float64 over K/V rows gathered through a page table; paged batch decode,
  split-K partials and their log-sum-exp merge, ragged and paged causal
  prefill.  ("FlashInfer parity matrix" page, section "Admitted attention
  matrix": rows Single decode split-K, Paged batch decode, Ragged causal
  prefill, Paged causal prefill; F32 softmax state, BF16, head dim 128,
  page size 16.)
* ``rope``: the NeoX split-half rotary embedding with explicit int32
  positions, and the fused RoPE + paged KV append into exclusively owned pages.
  (Same page, rows Standard RoPE and Fused RoPE plus paged append, and section
  "Paged KV ownership difference".)
* ``bf16``: exact bf16 -> float64 widening and float64 -> bf16 rounding
  (nearest, ties to even) in a single step.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*``
against facts that do not come from this package: torch's and scipy's library
routines on the special cases they cover, closed forms, invariances and
brute-force probes.  Readings of points the pages leave open are listed in the
docstrings of the functions they affect.
"""
