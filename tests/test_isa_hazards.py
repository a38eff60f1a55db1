"""Static check of the compiled kernels (CPU, no GPU needed): no vector read
of a matrix-core result closer to the MFMA that wrote it than the wait states
the compiler itself keeps, on any path through the control-flow graph.

gfx950 does not interlock a vector read (v_accvgpr_read of an AGPR, or any
VALU, LDS or store operand in a VGPR) against an in-flight MFMA writing the
register: the code must separate them by wait states.  Within a basic block
the compiler does; across a branch it once left three, and the read returned
the accumulator without the last products (wrong dK in one kernel, found by
the GPU parity tests).  This test compiles every kernel source to gfx950
assembly with the library's own flags, builds each function's basic blocks
and their predecessor edges (taken branches, fall-through into the next
block, loop back-edges), and for every vector read walks back along every
path to the nearest instruction that writes the register.  When that writer
is an MFMA, the wait states between the two (every issued instruction one,
branches included, ``s_nop N`` N + 1: the count LLVM's hazard recognizer
uses) must be at least what the compiler keeps inside a block.  Reads in
inline assembly are checked like any other.
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


MAX_NEED = 13
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
_NO_DEST = _STORES + ("global_load_lds", "buffer_load_lds", "s_")


def _reads(ins):
    """Registers a vector instruction reads (every operand of a store, every
    operand but the first otherwise).  MFMA operands are left out: chained
    products on one accumulator are forwarded in hardware."""
    if ins.startswith("s_") or ins.startswith("v_mfma"):
        return set()
    ops = _operands(ins)
    srcs = ops if ins.startswith(_STORES) else ops[1:]
    return set().union(*[_regs(o) for o in srcs]) if srcs else set()


def _writes(ins):
    """Registers an instruction writes (its first operand, for vector ALU,
    MFMA and load instructions)."""
    if ins.startswith(_NO_DEST):
        return set()
    ops = _operands(ins)
    return _regs(ops[0]) if ops else set()


def _states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def _is_label(line):
    return re.match(r"^\.LBB\S+:$", line) is not None


def _blocks(lines):
    """Basic blocks as (start, end) index ranges, a label -> block map and
    each block's predecessors."""
    starts = {0}
    for n, l in enumerate(lines):
        if _is_label(l):
            starts.add(n)
        if re.match(r"^s_(c?branch|setpc|endpgm)", l) and n + 1 < len(lines):
            starts.add(n + 1)
    starts = sorted(starts)
    blocks = [(s, e) for s, e in zip(starts, starts[1:] + [len(lines)])]
    at = {s: b for b, (s, _) in enumerate(blocks)}
    label_block = {lines[s][:-1]: b for b, (s, _) in enumerate(blocks) if _is_label(lines[s])}
    preds = {b: [] for b in range(len(blocks))}
    for b, (s, e) in enumerate(blocks):
        last = lines[e - 1]
        m = re.match(r"^s_(c?branch)\S*\s+(\.LBB\S+)", last)
        if m and m.group(2) in label_block:
            preds[label_block[m.group(2)]].append(b)
        falls = not re.match(r"^s_(branch|setpc|endpgm)", last)
        if falls and e in at:
            preds[at[e]].append(b)
    return blocks, preds


def short_mfma_reads(asm):
    """(function, line of the read, distance) for every vector read of a
    register that some path reaches from an MFMA writing it in fewer wait
    states than the compiler keeps within a block."""
    found = []
    for fm in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.find(".Lfunc_end", fm.end())
        lines = [l.split(";")[0].strip() for l in asm[fm.end():end].splitlines()]
        lines = [l for l in lines if l and not (l.startswith(".") and not _is_label(l))]
        blocks, preds = _blocks(lines)
        block_of = {}
        for b, (s, e) in enumerate(blocks):
            for n in range(s, e):
                block_of[n] = b

        def nearest(b, k, reg, dist, seen):
            """Smallest MFMA distance to `reg` before index k of block b."""
            s, _ = blocks[b]
            for n in range(k - 1, s - 1, -1):
                ins = lines[n]
                if _is_label(ins):
                    continue
                dist += _states(ins)
                if reg in _writes(ins):
                    return dist if ins.startswith("v_mfma") and dist < _need(ins) else None
                if dist >= MAX_NEED:
                    return None
            worst = None
            for p in preds[b]:
                if (p, dist) in seen:
                    continue
                seen.add((p, dist))
                d = nearest(p, blocks[p][1], reg, dist, seen)
                if d is not None and (worst is None or d < worst):
                    worst = d
            return worst

        for n, ins in enumerate(lines):
            for reg in _reads(ins):
                d = nearest(block_of[n], n, reg, _states(ins), set())
                if d is not None:
                    found.append((fm.group(1), n, d))
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

# the MFMA's block ends in a jump to a short trampoline block without MFMAs,
# which jumps on to the read
_TRAMPOLINE = """_Zkern:
  v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
  s_cbranch_scc1 .LBB0_3
  s_nop 7
  s_nop 7
  s_branch .LBB0_2
.LBB0_3:
  v_add_u32_e32 v9, v9, v9
  s_branch .LBB0_2
.LBB0_2:
  v_accvgpr_read_b32 v20, a3
  s_endpgm
.Lfunc_end0:
"""

# a read at the top of a loop whose last block ends in the MFMA
_LOOP = """_Zkern:
  v_mov_b32_e32 v30, 0
.LBB0_1:
  v_add_f32_e32 v31, v30, v18
  v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], v[16:31]
  s_cbranch_scc1 .LBB0_1
  s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_short_paths_and_accepts_padding():
    # the read is 4 states after the MFMA on the taken path, 5 on the fall-through
    bad = short_mfma_reads(_BAD)
    assert [d for _, _, d in bad] == [4], bad  # the shorter path is reported
    padded = _BAD.replace("  s_cbranch_scc1", "  s_nop 7\n  s_cbranch_scc1")
    assert short_mfma_reads(padded) == []
    other = _BAD.replace("v_accvgpr_read_b32 v20, a7", "v_accvgpr_read_b32 v20, a9")
    assert short_mfma_reads(other) == []
    # a result in VGPRs read by an ordinary VALU instruction
    vgpr = _BAD.replace("a[4:7], v[0:3], v[4:7], a[4:7]", "v[24:27], v[0:3], v[4:7], v[24:27]").replace(
        "v_accvgpr_read_b32 v20, a7", "v_add_f32_e32 v20, v26, v20")
    assert [d for _, _, d in short_mfma_reads(vgpr)] == [4]
    # a later write by another instruction ends the hazard
    overwritten = _BAD.replace("  ds_read_b128 v[10:13], v14", "  v_accvgpr_write_b32 a7, v14")
    assert short_mfma_reads(overwritten) == []


def test_checker_follows_trampolines_and_loop_back_edges():
    # the padded path is safe (1 + 1 + 16 + 1 + 1 = 20); the path through the
    # trampoline block is 1 + 1 + 1 + 1 + 1 = 5
    assert [d for _, _, d in short_mfma_reads(_TRAMPOLINE)] == [5]
    safe = _TRAMPOLINE.replace("  v_add_u32_e32 v9, v9, v9", "  v_add_u32_e32 v9, v9, v9\n  s_nop 15")
    assert short_mfma_reads(safe) == []
    # around the back-edge: MFMA, branch, the read at the top of the loop
    assert [d for _, _, d in short_mfma_reads(_LOOP)] == [3]
    assert short_mfma_reads(_LOOP.replace("  s_cbranch_scc1", "  s_nop 11\n  s_cbranch_scc1")) == []


def test_checker_sees_inline_assembly_reads():
    # an inline-assembly accumulator rescale (read, multiply, write back)
    # placed right after the product that wrote the register
    asm = """_Zkern:
  v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
  ;;#ASMSTART
  v_accvgpr_read_b32 v40, a5
  v_mul_f32 v40, v40, v41
  v_accvgpr_write_b32 a5, v40
  ;;#ASMEND
  s_endpgm
.Lfunc_end0:
"""
    assert [d for _, _, d in short_mfma_reads(asm)] == [2]


@pytest.mark.skipif(not os.path.exists(B._hipcc()), reason="hipcc not installed")
def test_compiled_kernels_have_no_short_mfma_reads():
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in SOURCES:
            out = os.path.join(tmp, src + ".s")
            cmd = [B._hipcc(), *[f for f in B.HIP_FLAGS if f != "-fPIC"], *B.FILE_FLAGS.get(src, []),
                   "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
            procs.append((src, out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE)))
        bad = []
        for src, out, p in procs:
            _, err = p.communicate(timeout=900)
            assert p.returncode == 0, err.decode()[-2000:]
            bad += [(src, *f) for f in short_mfma_reads(open(out).read())]
    assert not bad, bad
