"""CPU fp64 oracle of the TACT-KV codec -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product library never does.
"""
from .tact_oracle import *  # noqa: F401,F403
