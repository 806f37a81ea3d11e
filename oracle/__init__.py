"""CPU oracle for sorting-free categorical sampling.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from this
package.  The GPU library never calls it, links it or falls back to it, and
this package imports nothing from the GPU library: the two share no code.

Contents
--------
``philox``     Philox4x64-10 counter-based generator, written from its
               published definition (Salmon, Moraes, Dror, Shaw, "Parallel
               random numbers: as easy as 1, 2, 3", SC'11).
``reference``  sort-based filtering (top-k, top-p, min-p, top-k-then-top-p),
               the filtered target distribution, renormalisation, top-k
               logit masking and an exact inverse-transform (CDF) draw, all
               in exact rational arithmetic; plus a plain step-by-step model
               of dual-pivot rejection sampling and its exact output law on
               tiny vocabularies.

Every function cites the passage of the pages it follows.  Pins (tests that
tie the oracle to something other than itself) live in
``tests/test_oracle_pins.py``; every function listed above is pinned there.
"""
