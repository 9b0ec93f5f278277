"""Invariants of the kernels' inline assembly, checked on the gfx950 assembly the build flags
produce (CPU only: hipcc cross-compiles).

* The global->LDS copies (attention tiles, projection staging) set M0 inside inline assembly.
  That is safe only while the compiler itself keeps nothing in M0 in those kernels, so no
  compiler-generated instruction may name M0 in any kernel that issues such a copy.
* The nope output accumulators live in AGPRs written by inline-assembly MFMAs. Each attention
  kernel's descriptor must reserve the AGPRs it uses (next_free_vgpr - accum_offset), and the
  kernels make no calls (a callee would make the compiler save and restore live AGPRs).
"""
import os
import re
import shutil
import subprocess

import pytest

from segmented_attention_amd import build as B

HIPCC = B.HIPCC


def _asm(tmp_path, name="k_attn_mfma.hip"):
    src = os.path.join(B.CSRC, name)
    out = os.path.join(str(tmp_path), os.path.splitext(name)[0] + ".s")
    cmd = [HIPCC] + B.FLAGS + B.SOURCE_FLAGS.get(name, []) + [
        "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


def _functions(text):
    """name -> body lines of every kernel in an assembly listing."""
    funcs, name = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            funcs[name] = []
            continue
        if name is not None:
            if line.strip().startswith("s_endpgm"):
                name = None
                continue
            funcs[name].append(line)
    return funcs


def _compiler_m0_uses(lines):
    in_asm, bad = False, []
    for line in lines:
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0]
        if not in_asm and re.search(r"\bm0\b", code):
            bad.append(line.strip())
    return bad


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
def test_attention_kernel_asm_invariants(tmp_path):
    text = _asm(tmp_path)
    # split into functions; keep the attention kernels
    funcs = {}
    name = None
    for line in text.splitlines():
        m = re.match(r"^(_ZN6segmla11k_attn_mfma\S*):", line)
        if m:
            name = m.group(1)
            funcs[name] = []
            continue
        if name is not None:
            if line.strip().startswith("s_endpgm"):
                name = None
                continue
            funcs[name].append(line)
    assert len(funcs) == 4, sorted(funcs)

    for fname, lines in funcs.items():
        assert not any(re.search(r"\bs_(swappc|setpc|call)", l.split(";")[0]) for l in lines), fname
        in_asm = False
        for line in lines:
            if ";;#ASMSTART" in line:
                in_asm = True
                continue
            if ";;#ASMEND" in line:
                in_asm = False
                continue
            code = line.split(";")[0]
            if not in_asm and re.search(r"\bm0\b", code):
                pytest.fail("%s: compiler-generated instruction uses m0: %s" % (fname, line.strip()))

    # kernel descriptors: AGPRs reserved for the accumulators
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        kname, body = m.group(1), m.group(2)
        if "k_attn_mfma" not in kname:
            continue
        nfv = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        acc = int(re.search(r"\.amdhsa_accum_offset (\d+)", body).group(1))
        assert nfv - acc >= 256, (kname, nfv, acc)


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
def test_copy_kernels_keep_m0_free(tmp_path):
    """Every kernel with an inline-assembly global->LDS copy: no compiler-generated M0 use."""
    checked = 0
    for name in ("k_attn_mfma.hip", "k_epilogue.hip"):
        for fname, lines in _functions(_asm(tmp_path, name)).items():
            if not any("global_load_lds" in l for l in lines):
                continue
            checked += 1
            bad = _compiler_m0_uses(lines)
            assert not bad, (fname, bad[:3])
    assert checked >= 5, checked  # four attention instantiations + the projection
