"""fp64 CPU oracle for segment-relocated MLA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py. The library's product path never imports it.
"""
from . import segmla_oracle  # noqa: F401
