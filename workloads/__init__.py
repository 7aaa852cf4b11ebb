"""Seeded synthetic inputs for paged-KV POD attention.

This package only builds inputs: lengths, page tables and random values. It
holds none of the attention arithmetic, so both the fp64 oracle and the HIP
path can consume what it produces without sharing any of the method's code.
"""
from .configs import (  # noqa: F401
    RoleSpec,
    WorkloadSpec,
    Workload,
    RoleTensors,
    build,
    named_spec,
    NAMED,
    CascadeWorkload,
    build_cascade,
)
