"""Build libsegmla.so for gfx950 with hipcc (in-tree, next to this file).

Each HIP source is compiled to an object in parallel, then linked into one shared
library. Packed-FP32 instruction selection is disabled for all device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsegmla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["segmla_host.hip", "k_plan.hip", "k_attn_f32.hip", "k_attn_mfma.hip", "k_merge.hip",
           "k_epilogue.hip", "prefetch.hip"]

# The attention kernel keeps the score MFMAs in VGPR form (its nope output accumulators live
# in AGPRs, written by inline assembly), so it selects the VGPR MFMA form explicitly.
SOURCE_FLAGS = {"k_attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _compile(src, extra):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(extra_flags=(), jobs=None, verbose=False):
    """Compile every source and link libsegmla.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra_flags)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
