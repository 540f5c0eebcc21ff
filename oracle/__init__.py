"""CPU oracle for exact attention forward: test infrastructure, not product code.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
anything here. The GPU library never calls it and shares no code with it.

* ``oracle.exact``: the plain float64 definition (score matrix materialised,
  max-subtracted softmax, product with V, per-row log-sum-exp), the per-split
  form, the split reduction, and both over a paged K/V cache.
* ``oracle.backward``: the plain float64 gradient of the same definition (dQ,
  dK, dV for an upstream dO, by the chain rule through the materialised
  matrices), plus per-row and per-key samplers for long shapes.
* ``oracle.brute``: the same definition as scalar Python loops with ``math.fsum``,
  for tiny shapes only.
"""
from .exact import (attention, attention_rows, attention_split, combine,
                        softmax_rows, visible_mask, split_bounds, gather_paged,
                        attention_paged, attention_split_paged)
from .backward import attention_bwd, attention_bwd_dq_rows, attention_bwd_dkdv_cols

__all__ = ["attention", "attention_rows", "attention_split", "combine",
           "softmax_rows", "visible_mask", "split_bounds", "gather_paged",
           "attention_paged", "attention_split_paged", "attention_bwd",
           "attention_bwd_dq_rows", "attention_bwd_dkdv_cols"]
