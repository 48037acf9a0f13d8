"""Seeded synthetic inputs for the gated linear-attention workloads.

This module only draws random numbers and rounds them to the storage formats
the kernels read (bf16 by round-to-nearest-even).  It holds none of the
method's arithmetic: both the fp64 oracle and the HIP path consume the exact
host arrays produced here.
"""
from .inputs import *  # noqa: F401,F403
