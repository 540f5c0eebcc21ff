"""CPU oracle for exact attention forward: test infrastructure, not product code.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
anything here. The GPU library never calls it and shares no code with it.

* ``oracle.exact``: the plain float64 definition (score matrix materialised,
  max-subtracted softmax, product with V, per-row log-sum-exp), the per-split
  form and the split reduction.
* ``oracle.brute``: the same definition as scalar Python loops with ``math.fsum``,
  for tiny shapes only.
"""
from .exact import (attention, attention_rows, attention_split, combine,
                        softmax_rows, visible_mask, split_bounds)

__all__ = ["attention", "attention_rows", "attention_split", "combine",
           "softmax_rows", "visible_mask", "split_bounds"]
