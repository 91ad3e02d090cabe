"""Seeded synthetic inputs for block-sparse attention on flattened video layouts.

This package only builds inputs: token layouts cut into 128-row logical blocks,
sparse block graphs (the "selection" step that sits above the attention method)
and bf16 tensors.  It contains none of the attention or page-packing arithmetic,
so both the CPU oracle and the GPU path can consume the same inputs without
sharing any code under test.
"""
from .configs import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    make_workload,
    tile_layout,
)
