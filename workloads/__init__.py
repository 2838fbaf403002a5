"""Synthetic workloads (shape tables) and seeded input generators.

Shared by the oracle-side tests and the GPU path; contains no arithmetic of
the optimizer itself."""
from . import configs, gen  # noqa: F401
