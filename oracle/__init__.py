"""Plain, slow fp64 CPU oracle for the PISA piecewise sparse attention forward pass.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import, call or execute anything under ``oracle/``. The product path
(``libpisa`` and its Python binding) never imports it and shares no code, header, table or
helper with it; when the HIP library is missing the product path fails instead of falling back
here.

Modules:

* ``pisa_oracle`` - the method step by step in NumPy fp64 (statistics, routing, selection,
  piecewise numerator/denominator, normalisation) plus a dense-softmax reference.
* ``brute`` - pure-Python element loops (no NumPy) for tiny inputs: per-element Taylor
  expansion, block statistics and routing, used to pin ``pisa_oracle``.

Pin status per function (what fixes it other than itself) is stated in each docstring;
``routing_scores(..., routing="cov")`` - the covariance-aware score formula - is a reading of
the pages, not a printed formula: each of its terms is pinned by properties that fix it (listed in
its docstring), while the choice of formula itself is "parity unpinned".
"""

from . import brute, pisa_oracle  # noqa: F401
