"""fp64 CPU oracle for one rank's tensor-parallel shard (test infrastructure only).

Only tests, the smoke check and the benchmark's cpu_baseline leg may import it.
"""
from .tp_oracle import *  # noqa: F401,F403
