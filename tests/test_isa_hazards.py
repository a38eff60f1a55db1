"""Static check of the compiled kernels (CPU, no GPU needed): no read of a
matrix-core result right after a branch whose taken path leaves too few
wait states after the MFMA that wrote it.

gfx950 does not interlock a vector read (v_accvgpr_read of an AGPR, or any
VALU, LDS or store operand in a VGPR) against an in-flight MFMA writing the
register: the compiler must separate them by wait states.
Within a basic block it does; across a branch it once left three, and the read
returned the accumulator without the last products (wrong dK in one kernel,
found by the GPU parity tests).  This test compiles every kernel source to
gfx950 assembly with the library's own flags and measures, for every branch,
the wait states between the last MFMA of the branching block that writes a
register and the first read of that register at the branch target.
"""
import os
import re
import subprocess
import tempfile

import pytest

from causal_gqa_flashattention_amd import build as B

# Distance (instructions and s_nop wait states, from the MFMA to the read,
# both counted) that the compiler itself keeps inside a basic block on gfx950:
# 9 after a 16x16x32 product, 13 after a 32x32x16 one.
def _need(mfma):
    return 9 if "16x16" in mfma else 13


SCAN = 16  # instructions / wait states scanned at a branch target
SOURCES = ("fa_fwd.hip", "fa_bwd.hip", "fa_short.hip")


def _regs(tok):
    """Registers named by one operand, as ('a' | 'v', index) pairs."""
    m = re.match(r"([av])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(ins):
    return [o.strip().split()[0] for o in ins.split(None, 1)[1].split(",")] if " " in ins else []


_STORES = ("ds_write", "ds_store", "global_store", "buffer_store", "scratch_store", "flat_store")


def _reads(ins):
    """Registers a vector instruction reads (every operand of a store, every
    operand but the first otherwise)."""
    if ins.startswith("s_") or ins.startswith("v_mfma"):
        return set()
    ops = _operands(ins)
    srcs = ops if ins.startswith(_STORES) else ops[1:]
    return set().union(*[_regs(o) for o in srcs]) if srcs else set()


def _states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def short_branch_reads(asm):
    """(function, branch target, distance) for every accumulator read at a
    branch target closer to the MFMA that wrote it in the branching block
    than the compiler keeps within a block."""
    found = []
    for fm in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", fm.end())
        lines = [l.split(";")[0].strip() for l in asm[fm.end():end].splitlines()]
        lines = [l for l in lines if l]
        labels = {l[:-1]: n for n, l in enumerate(lines) if re.match(r"^\.LBB\S+:$", l)}
        # (instruction index the predecessor path ends at, target label): every
        # branch, and the fall-through into a label from a block that does
        # not end in an unconditional branch
        edges = []
        for n, ins in enumerate(lines):
            m = re.match(r"^s_c?branch\S*\s+(\.LBB\S+)", ins)
            if m and m.group(1) in labels:
                edges.append((n, m.group(1)))
            if n and re.match(r"^\.LBB\S+:$", ins) and not lines[n - 1].startswith("s_branch"):
                edges.append((n, ins[:-1]))
        for n, label in edges:
            reads, waited = {}, 0
            for k in range(labels[label] + 1, len(lines)):
                tgt = lines[k]
                if tgt.startswith(".LBB") or waited >= SCAN:
                    break
                waited += _states(tgt)
                for r in _reads(tgt):
                    reads.setdefault(r, waited)
            if not reads:
                continue
            back = 0
            for k in range(n - 1, -1, -1):
                src = lines[k]
                if src.startswith(".LBB"):
                    break
                back += _states(src)
                if src.startswith("v_mfma"):
                    hit = [w for r, w in reads.items() if r in _regs(_operands(src)[0])]
                    if hit:
                        if back + min(hit) < _need(src):
                            found.append((fm.group(1), label, back + min(hit)))
                        break
                if back > 64:
                    break
    return found


_BAD = """_Zkern:
  v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], a[4:7]
  s_cbranch_scc1 .LBB0_2
  v_add_u32_e32 v9, v9, v9
.LBB0_2:
  ds_read_b128 v[10:13], v14
  v_accvgpr_read_b32 v20, a7
  s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_a_short_path_and_accepts_padding():
    # the branch path (3) and the fall-through path (5) are both short
    assert short_branch_reads(_BAD) == [("_Zkern", ".LBB0_2", 3), ("_Zkern", ".LBB0_2", 5)]
    padded = _BAD.replace("  s_cbranch_scc1", "  s_nop 7\n  s_nop 3\n  s_cbranch_scc1")
    assert short_branch_reads(padded) == []
    other = _BAD.replace("v_accvgpr_read_b32 v20, a7", "v_accvgpr_read_b32 v20, a9")
    assert short_branch_reads(other) == []
    # a result in VGPRs read by an ordinary VALU instruction
    vgpr = _BAD.replace("a[4:7], v[0:3], v[4:7], a[4:7]", "v[24:27], v[0:3], v[4:7], v[24:27]").replace(
        "v_accvgpr_read_b32 v20, a7", "v_add_f32_e32 v20, v26, v20")
    assert short_branch_reads(vgpr) == [("_Zkern", ".LBB0_2", 3), ("_Zkern", ".LBB0_2", 5)]


@pytest.mark.skipif(not os.path.exists(B._hipcc()), reason="hipcc not installed")
def test_compiled_kernels_have_no_short_accumulator_reads_after_branches():
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in SOURCES:
            out = os.path.join(tmp, src + ".s")
            cmd = [B._hipcc(), *[f for f in B.HIP_FLAGS if f != "-fPIC"], *B.FILE_FLAGS.get(src, []),
                   "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
            procs.append((src, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE)))
        bad = []
        for src, out, p in procs:
            _, err = p.communicate(timeout=600)
            assert p.returncode == 0, err.decode()[-2000:]
            bad += [(src, *f) for f in short_branch_reads(open(out).read())]
    assert not bad, bad
