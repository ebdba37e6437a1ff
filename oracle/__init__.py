"""CPU oracle for the ZeRO shard step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and shares no code with
it: this package re-derives every result from the pages in plain NumPy.

What it computes, and where the pages state it:

* ``layout``     -- the flat parameter vector split into N equal contiguous
  shards, zero-padded to a multiple of N when asked ("ZeRO and FSDP",
  "Implementing ZeRO's Adam from scratch"; "The four schemes", ``Base``), and
  the per-unit split of ZeRO-3 ("ZeRO and FSDP", "ZeRO-3 and FSDP").
* ``numerics``   -- the rank-order fp32 reduce of 16-bit gradients, the
  mixed-precision Adam update with bias correction and eps outside the square
  root ("The four schemes", ``Base._adam``; "ZeRO and FSDP", ``ZeroAdam.step``),
  and the fp32 -> 16-bit round-to-nearest-even cast of the working copy.
* ``accounting`` -- resident bytes per band, the ZeRO-3 peak and per-rank
  traffic in elements and bytes ("The four schemes", accounting methods and
  the resident-vs-peak table; "ZeRO, annotated" section 5 and section 7;
  "One Poem Suffices: ZeRO" section 4.1; "Sharding the States.").
* ``schemes``    -- data parallel, ZeRO-1, ZeRO-2 and ZeRO-3 over N simulated
  ranks, including ZeRO-3's per-unit gather -> use -> release -> re-gather
  schedule with counters.
* ``sampled``    -- the per-element trajectory of any set of parameter
  indices, for checks at sizes where the whole vector is too large for NumPy.

Precision: the pages fix it (fp32 master, m and v; 16-bit parameters and
gradients), so the oracle computes in fp32 with one NumPy operation per
arithmetic step and no fused multiply-add.  Every function is pinned by
``tests/test_oracle_*.py`` against values printed on the pages, closed forms,
library routines (torch casts, ``torch.optim.Adam``) or brute force.

Parity unpinned: the default owner of a unit of unequal size under owner
broadcast (``layout.unit_owners`` on unequal units).  The pages show only
equal partitions, where the rule is pinned; for unequal units it is a
reading (the unit's midpoint decides) that no passage fixes.  An explicit
owner map (``make_layout(..., owners=...)``) avoids the reading: the tests
that run unequal units on the GPU pass one.
"""
