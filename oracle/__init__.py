"""CPU oracle for the TurboQuant KV-cache path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .tq_oracle import *  # noqa: F401,F403
