"""Seeded synthetic inputs for the NVFP4 sparse-MLA path.

This package only draws random numbers and lays them out (pool values,
queries, index lists, block tables).  It holds none of the method's
arithmetic: no quantisation, no decoding, no attention.  Both the oracle
side and the HIP side of every test and of the benchmark take their inputs
from here, and from nowhere else.
"""

from .workloads import (  # noqa: F401
    Workload, WORKLOAD_NAMES, make_workload, make_custom, pool_values, SM_SCALE,
)
