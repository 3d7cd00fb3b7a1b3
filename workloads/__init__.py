"""Seeded synthetic attention-layer inputs shared by the tests, the benchmark and the oracle checks.

This package synthesises Q, K and V only. It holds none of the attention method's arithmetic
(no block statistics, no scores, no selection, no softmax).
"""

from .gen import WORKLOADS, Workload, custom, workload, head_inputs, layer_inputs, to_float64  # noqa: F401
