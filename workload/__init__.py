"""Seeded synthetic inputs for the decode-attention workloads.

Shared by the oracle side (host, ``recipe``) and the device side (``device``,
fill kernels in ``csrc/fill.hip``).  It draws numbers only; it holds none of the
attention method's arithmetic.
"""
from .configs import STACKS, WORKLOADS, Workload, get  # noqa: F401
from .recipe import Recipe, recipe_for  # noqa: F401
