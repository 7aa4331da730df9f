"""CPU oracle for the WildCat hot path: plain, slow, float64 — TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of bench.py may import
this package.  The product path (the HIP library and its Python binding) never imports,
links or calls anything here, and this package imports nothing from the product path.

Modules:
  * ``wildcat``: initial residual, pivot sampling, randomly pivoted Cholesky, Nystroem
    weights, coreset attention, exact softmax attention, forced-uniform snapping.
  * ``philox``: the Philox4x64-10 generator the pivot draws come from.

Every function is pinned by the tests in tests/test_oracle_*.py to facts the pages or the
mathematics fix (full-rank reconstruction, the Nystroem identity, closed forms at r = 1 and
r = n, interpolation at the pivot keys, invariances of exact attention, numpy's own Philox
bit generator, distribution of the first pivot).
"""
from . import philox, wildcat  # noqa: F401
