"""Seeded synthetic inputs for the NVFP4 sparse-MLA path.

This package only draws random numbers and lays them out (pool values,
queries, index lists, block tables, indexer keys and queries).  It holds
none of the method's arithmetic: no quantisation of the cache rows, no
decoding, no attention, no scoring or selection.  Indexer keys and queries
are inputs stored as E4M3 bytes; they are drawn as N(0,1) values and cast by
torch's own float8_e4m3fn conversion.  Both the oracle
side and the HIP side of every test and of the benchmark take their inputs
from here, and from nowhere else.
"""

from .workloads import (  # noqa: F401
    Workload, WORKLOAD_NAMES, make_workload, make_custom, pool_values, SM_SCALE,
    IndexerInputs, indexer_inputs, fp8_values,
)
