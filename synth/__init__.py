"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

Holds shapes and random-number generation only; none of the method's
arithmetic lives here.
"""
from .configs import Workload, WORKLOADS, TINY, DFLASH, DSPARK, LONGCTX, HIGHBATCH, MEDIUM
from . import rng, inputs

__all__ = ["Workload", "WORKLOADS", "TINY", "DFLASH", "DSPARK", "LONGCTX", "HIGHBATCH",
           "MEDIUM", "rng", "inputs"]
