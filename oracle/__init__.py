"""CPU oracle for packed, block-causal varlen attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``packed_varlen_block_amd``) and imports nothing from it.

Everything here is plain and slow on purpose: float64 numpy, definitional
loops, one segment and one head at a time, written from the pages

* "Packing与 FlashAttention Varlen" (sections 1-5): the flat token axis, the
  cu_seqlens boundary, local position_ids and causal-inside-a-slice semantics;
* "Pack sequences without joining their contexts": the capacity-6 next-fit
  example, the block-causal permission rule and the constructed loss probe.

Modules
  packing     -- O1 metadata, O2 next-fit, O3 best-fit-decreasing, O4 pair forming,
                 O9 boundaries compiled back from position ids
  attention   -- O5 forward, O6 backward, O7 brute-force dense masked attention
  loss_probe  -- O8 the constructed loss probe, O10 the packed-row loss
  linear_attention -- O11 the gated delta rule with its state reset at every boundary

Parity status: every function here is pinned by tests under ``tests/``
(``-m "not gpu"``) against values the pages print, closed forms, brute force
or library routines.  The best-fit-decreasing tie-breaks are a reading (the
pages name the policy only); they are pinned by hand-worked cases and a
definitional replay check.
"""
