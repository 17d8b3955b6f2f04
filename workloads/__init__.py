"""Seeded synthetic workloads for batched speculative verification.

This package is shared by the tests, the benchmark and the oracle's callers.
It draws random numbers and encodes them in the storage formats the library
consumes (bf16, int4 groups of 32 with bf16 scales).  It holds none of the
verification arithmetic itself: no normalisation, projection, attention,
acceptance test or sampling rule lives here.
"""
from .gen import *  # noqa: F401,F403
from .configs import *  # noqa: F401,F403
