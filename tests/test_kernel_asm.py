"""Invariants of the attention kernel's inline assembly, checked on the gfx950 assembly the
build flags produce (CPU only: hipcc cross-compiles).

* The global->LDS copies set M0 inside inline assembly. That is safe only while the compiler
  itself keeps nothing in M0 in these kernels, so no compiler-generated instruction may name
  M0.
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


def _asm(tmp_path):
    src = os.path.join(B.CSRC, "k_attn_mfma.hip")
    out = os.path.join(str(tmp_path), "k_attn_mfma.s")
    cmd = [HIPCC] + B.FLAGS + B.SOURCE_FLAGS.get("k_attn_mfma.hip", []) + [
        "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


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
