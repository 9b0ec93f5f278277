"""segmented_attention_amd: segment-relocated MLA attention for AMD MI355X (gfx950).

The compute path is libsegmla.so (hand-written HIP kernels behind the C ABI in
include/segmla.h); `segmla` is its ctypes binding.
"""
from . import segmla  # noqa: F401
from .segmla import Plan, SegmlaError  # noqa: F401
