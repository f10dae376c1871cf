"""CPU oracle for the sharded matmul A[I,J].B[J,K] -> C[I,K].

TEST INFRASTRUCTURE ONLY. This package may be imported, called, linked or
executed only by the test-suite (``tests/``), by the smoke check in
``__graft_entry__.py`` and by the CPU-baseline leg of ``bench.py``. The HIP
library and its Python binding never import it, and it never imports them:
the two sides share no code, headers, tables or helpers. Only the seeded
input generators in ``workloads`` serve both.

Contents
  * ``oracle.c``  -- naive fp64 loops (products, entries, mat-vec, rank-order
    sums, GeLU(tanh), fp64 -> bfloat16 rounding), built to ``liboracle.so``.
  * ``planner``   -- reference planner (four cases, shard coordinates).
  * ``reference`` -- the method's outputs composed from the two: per-unit
    partials, group sums, all-reduce / reduce-scatter / all-gather
    ownership, the dense product, the MLP chain.

Parity status of each function is stated in ``reference``'s docstring.
"""
from .build import load_library  # noqa: F401
