"""Seeded synthetic inputs for the sparse-attention decode path.

This package only draws random numbers and lays them out in the paged
formats the kernels and the oracle both read. It holds none of the method's
arithmetic (no scores, no selection, no attention), so either side can use it
without sharing code with the other.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    Inputs,
    make_inputs,
    small_variant,
    host_view,
    raw_numpy,
    PagedRows,
    to_device,
    locality_indices,
)
