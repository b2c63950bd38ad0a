"""Synthetic workloads shared by the tests and the benchmark.

* ``generate``   -- seeded input generators (random numbers only; none of the
  method's arithmetic).  The one module both the HIP path's tests and the
  oracle's tests take inputs from.
* ``configs``    -- the named problem shapes (tiny check, base encoder, base
  decoder block, big cross-attention, long causal, and the L >= 1024 sweep).
* ``accounting`` -- algorithmic FLOP and byte counts per workload.
"""
