"""CPU oracle for the attention forward pass.  TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 implementation of what the GPU path
computes, used to check it.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and this
package imports nothing from the library.

* :mod:`oracle.ref`  -- numpy: the plain definition, a tile-by-tile online
  softmax, ragged batches, decode and split-KV decode with its merge.
* :mod:`oracle.cpu`  -- the same plain definition as C loops (``oracle_cpu.c``)
  with OpenMP, for spot checks of the large workloads and the CPU baseline.

Every function is pinned by tests against closed forms, invariants, a
50-digit brute force and special cases (tests/test_oracle.py).
"""
