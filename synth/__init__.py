"""Seeded synthetic workloads for MLA decode (shared by the oracle-side tests and the GPU path).

This package only draws random numbers, casts them to storage types and lays them out
(contiguous rows, paged pools, block tables). It holds none of the method's arithmetic:
no projection, no rotary embedding, no quantisation and no attention.
"""
from .configs import CONFIGS, Dims, RUNNING_DIMS, V2_DIMS, get_config  # noqa: F401
from .gen import Case, make_case, make_prefill_case  # noqa: F401
