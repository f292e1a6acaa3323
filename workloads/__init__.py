"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package holds the five workload shapes and the seeded generators of their
inputs (queries, keys, values, token ids and the Gaussian sketch projection).
It holds none of the method's arithmetic: no attention, no scoring, no
eviction.  Both the CPU oracle's callers and the GPU path's callers draw their
inputs from here, so both sides always see the same rounded tensors.
"""

from .configs import WORKLOADS, Workload, get, scaled  # noqa: F401
from .generate import LayerInputs, generate_layer, unit_sequence  # noqa: F401
