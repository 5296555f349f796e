"""CPU fp64 oracle of MALA: test infrastructure, never part of the product path.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .mala_oracle import *  # noqa: F401,F403
