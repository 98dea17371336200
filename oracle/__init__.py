"""CPU oracle for Sketch Attention (SA) — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct float64 reference that the
HIP path is checked against.  Nothing in the product path may import, call,
link or execute it: only the tests, the smoke check of the build entry module
and the CPU-baseline leg of the benchmark use it.  It shares no code, tables
or helpers with the HIP library and imports nothing from the product package.

Sources (the method's definition):
  * "SequenceO1: End-to-End Ultra-Long (100K) Sequence Modeling in
    Recommendation with Low-Rank Caching", reading notes page
    (paper-archivist.com), section 3.1, Eq. (5)-(9): prototypes, affinities,
    prototype-wise softmax, sketch aggregation.
  * The same paper's HTML page (arXiv 2609.08443), the FlashSA paragraph of the
    system-design section: streaming max / log-sum-exp statistics, no k x n
    matrix kept.
  * Reading notes, section 5 (appendix G), Eq. (23)-(36): analytic FLOP counts.

Modules
  sa_ref  -- numpy float64 forward / backward over a CSR-ragged batch.
  brute   -- pure-Python scalar loops (math.fsum) for tiny inputs.
  flops   -- the pages' analytic FLOP formulas, Eq. (23)-(36).

Parity status: every function here is pinned by a CPU test under tests/ (see
the header of each module for its pins); none is "parity unpinned".
"""
