"""Float64 CPU oracle of the SWAN hybrid-cache decode step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .oracle import (OracleCache, attend, build, default_threads, lib, project, prune, rope,  # noqa: F401
                     round_e4m3, round_f16)
