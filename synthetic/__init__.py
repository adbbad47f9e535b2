"""Seeded synthetic workloads for the two-sided rounding problem.

This package only *generates inputs* (weight matrices, SPD metric matrices and
per-row grid scales).  It holds none of the rounding method's arithmetic, so the
CPU oracle and the GPU library can both consume its arrays without sharing any
code of the method itself.
"""
from .configs import (  # noqa: F401
    CONFIG_NAMES, SHAPES3, Workload, Workload3, make, make3, make_conditioned, make_powerlaw,
    make_random, make_random3)
