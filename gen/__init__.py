"""Seeded synthetic inputs for draft-tree verification.

This package is shared by the tests, the benchmark and the smoke check. It
produces inputs only: random tensors, random tree topologies, synthetic
per-depth draft candidate lists and target logits (with optional planting of
the greedy token). It performs none of the verification arithmetic (no
attention, no argmax, no acceptance walk, no best-first tree build); those live
in the library under test and, independently, in the oracle.

Every generator takes a ``numpy.random.Generator`` (PCG64) obtained from
:func:`gen.rng.stream`, so a workload is a pure function of its seed.
"""

from .rng import stream  # noqa: F401
from . import trees, draft, tensors, configs  # noqa: F401
