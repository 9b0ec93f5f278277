"""Seeded synthetic workloads for segment-relocated MLA attention.

This package only describes request shapes and draws random tensors. It holds
none of the method's arithmetic: no rotation, attention, selection or
projection. Both the HIP path (through its tests and the bench) and the fp64
oracle consume exactly the tensors produced here.
"""
from .configs import CONFIGS, SMALL_CONFIGS, config_by_name, segment_table  # noqa: F401
from .gen import make_inputs, make_dual_inputs, SEG_PREFIX, SEG_DOC, SEG_NEW  # noqa: F401
