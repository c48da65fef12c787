"""Seeded synthetic workloads (shapes + input generators) shared by tests and bench.

Holds none of the method's arithmetic; see ``generate.py`` for the input recipe.
"""

from .configs import WORKLOADS, Workload, ConfClass, get  # noqa: F401
from .generate import Inputs, paged_cache  # noqa: F401
