"""Invariants of the kernels' inline assembly, checked on the gfx950 assembly the build flags
produce (CPU only: hipcc cross-compiles).

* The global->LDS copies (attention tiles, projection staging) set M0 inside inline assembly.
  That is safe only while the compiler itself keeps nothing in M0 in those kernels, so no
  compiler-generated instruction may name M0 in any kernel that issues such a copy.
* The nope output accumulators live in AGPRs written by inline-assembly MFMAs. Each attention
  kernel's descriptor must reserve the AGPRs it uses (next_free_vgpr - accum_offset), and the
  kernels make no calls (a callee would make the compiler save and restore live AGPRs).
* An MFMA must not read a register that the vector ALU wrote less than two wait states
  before. The compiler keeps this for its own MFMAs; the inline-assembly MFMAs without their
  own s_nop rely on their operands coming from LDS reads, which is checked here instruction
  by instruction.
"""
import os
import re
import shutil
import subprocess

import pytest

from segmented_attention_amd import build as B

HIPCC = B.HIPCC


_ASM_CACHE = {}


def _asm(tmp_path, name="k_attn_mfma.hip"):
    """gfx950 assembly of one source with the build's flags (compiled once per test session:
    the attention source takes about 40 s)."""
    if name not in _ASM_CACHE:
        src = os.path.join(B.CSRC, name)
        out = os.path.join(str(tmp_path), os.path.splitext(name)[0] + ".s")
        cmd = [HIPCC] + B.FLAGS + B.SOURCE_FLAGS.get(name, []) + [
            "--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        _ASM_CACHE[name] = open(out).read()
    return _ASM_CACHE[name]


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
        m = re.match(r"^(_ZN6segmla(?:11k_attn_mfma|10k_attn_dec)\S*):", line)
        if m:
            name = m.group(1)
            funcs[name] = []
            continue
        if name is not None:
            if line.strip().startswith("s_endpgm"):
                name = None
                continue
            funcs[name].append(line)
    # (v_has_rope, E4M3, sink + window) instantiations, and the decode kernel's six (v_has_rope
    # x split decode, every available compressed entry, listed entries)
    assert len(funcs) == 14, sorted(funcs)

    for fname, lines in funcs.items():
        # no calls (s_setpc alone is also the far-jump form of a branch in a large kernel)
        assert not any(re.search(r"\bs_(swappc|call)", l.split(";")[0]) for l in lines), fname
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
        if "k_attn_mfma" not in kname and "k_attn_dec" not in kname:
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


_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+))")


def _regs(text):
    """Set of ('v'|'a', index) named by an operand list."""
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        lo = int(m.group(2) if m.group(2) is not None else m.group(4))
        hi = int(m.group(3) if m.group(3) is not None else m.group(4))
        out.update((kind, r) for r in range(lo, hi + 1))
    return out


def _valu_mfma_hazards(lines, window=2):
    """Inline-assembly MFMAs (AGPR accumulators) issued without an s_nop of their own, where
    a vector-ALU instruction within `window` wait states before names one of the MFMA's
    registers (conservative: any register operand of the VALU instruction counts as written).
    A label inside the window counts as a hazard (another path may reach the MFMA)."""
    bad, prev = [], []  # prev: (kind, wait_states, mnemonic, operands) most recent last
    in_asm, asm_first = False, False
    for line in lines:
        t = line.strip()
        if ";;#ASMSTART" in t:
            in_asm, asm_first = True, True
            continue
        if ";;#ASMEND" in t:
            in_asm = False
            continue
        if t.startswith(".LBB") or t.startswith("; %bb."):
            prev.append(("label", 1, "", ""))
            continue
        code = t.split(";")[0].strip()
        if not code or code.startswith("."):
            continue
        mnem, _, ops = code.partition(" ")
        if in_asm and mnem.startswith("v_mfma") and "a[" in ops and asm_first:
            need, seen = window, 0
            for kind, ws, pm, pops in reversed(prev):
                if seen >= need:
                    break
                if kind == "label":
                    bad.append(("label before", code))
                    break
                if pm.startswith("v_") and not pm.startswith("v_mfma") and _regs(pops) & _regs(ops):
                    bad.append((pm + " " + pops, code))
                    break
                seen += ws
        if in_asm:
            asm_first = False
        ws = 1
        m = re.match(r"s_nop (\d+)", code)
        if m:
            ws = int(m.group(1)) + 1
        prev.append(("insn", ws, mnem, ops))
        if len(prev) > 16:
            prev.pop(0)
    return bad


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
def test_assembly_mfmas_without_nop_read_no_fresh_valu_result(tmp_path):
    funcs = {k: v for k, v in _functions(_asm(tmp_path)).items() if "k_attn_mfma" in k or "k_attn_dec" in k}
    assert len(funcs) == 14, sorted(funcs)  # 8 prefill instantiations + 6 decode-kernel modes
    checked = 0
    for fname, lines in funcs.items():
        bad = _valu_mfma_hazards(lines)
        assert not bad, (fname, bad[:3])
        checked += sum(1 for l in lines if re.match(r"\s*v_mfma\S* a\[", l))
    assert checked >= 4 * 16, checked


def test_hazard_checker_flags_a_fresh_valu_write():
    """The checker itself: a VALU write of an operand right before a nop-less MFMA is found,
    the same write three instructions earlier is not."""
    mf = ["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[72:75], v[68:71], a[0:15]", "\t;;#ASMEND"]
    near = ["\tv_add_u32_e32 v73, s0, v94", "\ts_waitcnt lgkmcnt(2)"] + mf
    far = ["\tv_add_u32_e32 v73, s0, v94", "\tds_read_b64_tr_b16 v[80:81], v95", "\ts_waitcnt lgkmcnt(2)"] + mf
    other = ["\tv_add_u32_e32 v90, s0, v94", "\ts_waitcnt lgkmcnt(2)"] + mf
    label = ["\tds_read_b64_tr_b16 v[80:81], v95", ".LBB1_5:", "\ts_waitcnt lgkmcnt(2)"] + mf
    nop = ["\tv_add_u32_e32 v73, s0, v94", "\t;;#ASMSTART", "\ts_nop 1",
           "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[72:75], v[68:71], a[0:15]", "\t;;#ASMEND"]
    assert _valu_mfma_hazards(near)
    assert not _valu_mfma_hazards(far)
    assert not _valu_mfma_hazards(other)
    assert _valu_mfma_hazards(label)
    assert not _valu_mfma_hazards(nop)


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
def test_decode_kernel_keeps_everything_in_registers(tmp_path):
    """The decode kernel holds 256 accumulator values, 29 query steps and its operand rings per
    lane: any private (scratch) memory would mean spilled accumulators or query fragments. The
    same holds for its two-pool modes (every available entry, listed entries)."""
    text = _asm(tmp_path)
    found = 0
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        if "k_attn_dec" not in m.group(1):
            continue
        found += 1
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2)).group(1))
        assert priv == 0, (m.group(1), priv)
    assert found == 6, found


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
def test_attention_key_loops_do_not_spill(tmp_path):
    """The prefill attention instantiations hold 256 accumulator values and the query in
    registers; a change that tips the key loop into spilling (the E4M3 variant once spilled 152
    bytes inside it and ran 7.5 % slower) shows up as scratch accesses between the loop's
    barriers. A few values spilled around the loop (prologue, epilogue, rare out-of-line paths)
    cost nothing measurable; the total private memory stays small."""
    text = _asm(tmp_path)
    funcs = {k: v for k, v in _functions(text).items() if "k_attn_mfma" in k}
    assert len(funcs) == 8, sorted(funcs)
    for fname, lines in funcs.items():
        bars = [i for i, l in enumerate(lines) if l.strip().startswith("s_barrier")]
        assert len(bars) >= 7, (fname, len(bars))
        loop = lines[bars[2]:bars[6]]  # steady-state iterations of the unrolled key loop
        bad = [l.strip() for l in loop if l.strip().startswith("scratch_")]
        assert not bad, (fname, bad[:3])
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        if "k_attn_mfma" in m.group(1):
            priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2)).group(1))
            assert priv <= 64, (m.group(1), priv)
