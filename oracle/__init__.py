"""CPU float64 oracle for exact attention (test infrastructure only).

Nothing in the product path may import this package. Only the test suite,
the smoke check in the graft entry module, and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library: it is written from the
definition of scaled-dot-product attention, materialises the full score
matrix, and uses numpy (BLAS) matmuls as its only library primitive.

Modules:
  attention  full-matrix numpy implementation: masks, forward, varlen,
             split-KV partials and their combine, paged gather, paged prefill
             and paged decode, the backward (dQ, dK, dV) for dense and packed
             sequences,
             and a per-row evaluator for sampling very large problems.
  brute      scalar Python loops over (batch, head, query, key, dim) for
             tiny shapes; an independent second reading of the definition.
"""
from . import attention, brute  # noqa: F401
