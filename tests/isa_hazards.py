"""Wait-state checks on the gfx950 assembly of the kernels (used by
test_isa_hazards.py; CPU only).

The GEMM engine issues its MFMAs as inline asm (tied accumulators), and the
compiler's hazard recognizer does not look inside asm: the code keeps the
required distances itself (s_nop drains before accumulators are read, two
wait states before the first MFMA that reads a fragment rewritten by VALU
code).  This scans the instruction stream of each kernel, straight through
branches (conservative), and reports
  * a VALU instruction that writes a VGPR (or AGPR) which an MFMA then reads
    as a source operand fewer than `valu_to_mfma` wait states later;
  * a non-MFMA instruction that reads an AGPR (or VGPR) an MFMA wrote fewer
    than `mfma_to_read` wait states earlier (an MFMA accumulating into the
    same registers is interlocked by the hardware and exempt).
Wait states are counted as one per instruction and N + 1 per s_nop N.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"^([av])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"^([av])(\d+)$")


def regs(op: str):
    op = op.strip()
    m = _RANGE.match(op)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(op)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def instructions(asm: str):
    """(kernel, opcode, operands) in program order, kernels from their labels."""
    func = None
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        if not line or line.startswith(".") and not line.startswith(".LBB"):
            continue
        if line.endswith(":"):
            if not line.startswith(".L"):
                func = line[:-1]
            continue
        parts = line.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        yield func, parts[0], ops


def check(asm: str, kernel_filter=lambda name: True, valu_to_mfma: int = 2,
          mfma_to_read: int = 18):
    problems = []
    recent_valu = []   # [wait states ago, registers written]
    recent_mfma = []
    func = None
    for f, opc, ops in instructions(asm):
        if f != func:
            func, recent_valu, recent_mfma = f, [], []
        if not func or not kernel_filter(func):
            continue
        if opc.startswith("v_mfma"):
            srcs = set()
            for o in ops[1:3]:
                srcs |= regs(o)
            acc = regs(ops[3]) if len(ops) > 3 else set()
            for ago, r in recent_valu:
                if ago < valu_to_mfma and (r & (srcs | acc)):
                    problems.append(f"{func}: VALU write of {sorted(r & (srcs | acc))} {ago} wait "
                                    f"states before {opc} {', '.join(ops)}")
            ws = 1
        else:
            ws = int(ops[0], 0) + 1 if opc == "s_nop" and ops else 1
            reads = set()
            for o in ops[1:] if opc.startswith("v_") else ops:
                reads |= regs(o)
            # stores read their data operand; loads and DS reads only write
            if opc.startswith(("buffer_load", "global_load", "ds_read", "flat_load")):
                reads = set()
            for ago, r in recent_mfma:
                if ago < mfma_to_read and (r & reads):
                    problems.append(f"{func}: {opc} reads {sorted(r & reads)} {ago} wait states "
                                    f"after an MFMA wrote it")
        recent_valu = [(a + ws, r) for a, r in recent_valu if a + ws < 64]
        recent_mfma = [(a + ws, r) for a, r in recent_mfma if a + ws < 64]
        if opc.startswith("v_mfma"):
            recent_mfma.append((0, regs(ops[0])))
            # an MFMA that accumulates into registers other MFMAs are still
            # writing is interlocked: only non-MFMA readers are checked
        elif opc.startswith("v_") and ops:
            recent_valu.append((0, regs(ops[0])))
    return problems
