"""Wait-state check of the generated gfx950 code.

Several MFMAs in the decode kernels are issued as inline assembly (to keep
the accumulators pinned in their registers).  The compiler does not see
those MFMAs, so it cannot insert the wait states the matrix cores require
around them; the kernels insert what they know they need, and this check
verifies the final instruction stream instead of trusting that:

  * VALU write of a VGPR/AGPR -> MFMA read of it: at least 2 wait states;
  * MFMA write -> VALU (or v_accvgpr_read) read of the result, or a VALU
    write of the same registers: at least 12 wait states after an 8-pass
    v_mfma_f32_32x32x16_bf16 and 20 after a 16-pass
    v_mfma_f32_32x32x64_f8f6f4 (any other MFMA: 20).  These are the counts
    hipcc inserts for gfx950 after its own MFMAs (an MFMA builtin followed
    by a VALU read of the result compiles to s_nop 11, resp. s_nop 15 +
    s_nop 3);
  * f8f6f4 MFMA read of a source (A, B or C operand) -> VALU write of it: at
    least 4 wait states (measured: a VALU write one wait state after such an
    MFMA gave wrong results, three and more did not; bf16 MFMAs read their
    operands at issue, and the kernels overwrite them right after without
    error);

where `s_nop N` counts N + 1 wait states and every other instruction one.
Used by build.py on every kernel in the device assembly of the kernels source.

Limits of the check (what it does not prove):
  * it scans each function's text straight backwards from an instruction and
    ignores control flow, so a hazard across a branch or a loop back edge
    (a read at the top of a loop of a result written at its bottom) is not
    seen;
  * it treats only VALU instructions (v_* other than MFMAs) as readers or
    writers: DS / buffer / global stores that read an MFMA destination, and
    loads that overwrite an MFMA operand, are not modelled;
  * it knows the result latencies of the two MFMA opcodes the kernels
    issue; any other MFMA gets the larger one.
The kernels therefore do not rely on it alone: every inline-assembly MFMA
chain ends with an explicit s_nop drain of at least its opcode's count
before any other instruction can read its results, on every path.
"""
from __future__ import annotations

import re
import sys

VALU_TO_MFMA = 2
MFMA_TO_VALU = {"v_mfma_f32_32x32x16_bf16": 12, "v_mfma_f32_32x32x64_f8f6f4": 20}
MFMA_TO_VALU_DEFAULT = 20
MFMA_SRC_TO_VALU_WRITE = 4


def _mfma_to_valu(op: str) -> int:
    return MFMA_TO_VALU.get(op, MFMA_TO_VALU_DEFAULT)


def _regs(tok: str):
    tok = tok.strip()
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _instructions(lines):
    out = []
    for raw in lines:
        line = raw.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        out.append(line)
    return out


def _operands(line: str):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in parts[1].split(",")]


def _ws(line: str) -> int:
    op, ops = _operands(line)
    if op == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def check_function(lines, name=""):
    """Return a list of violation strings for one function body."""
    ins = _instructions(lines)
    bad = []
    for i, line in enumerate(ins):
        op, ops = _operands(line)
        if op.startswith("v_mfma"):
            srcs = set().union(*[_regs(o) for o in ops[1:4]]) if len(ops) >= 4 else set()
            ws, j = 0, i - 1
            while j >= 0 and ws < VALU_TO_MFMA:
                pop, pops = _operands(ins[j])
                if pop.startswith("v_") and not pop.startswith("v_mfma") and pops:
                    if _regs(pops[0]) & srcs:
                        bad.append(f"{name}: VALU write {ins[j]!r} -> {line!r} after {ws} wait states")
                ws += _ws(ins[j])
                j -= 1
        elif op.startswith("v_") and ops:
            reads = set().union(*[_regs(o) for o in ops[1:]])
            if op.startswith("v_accvgpr_read"):
                reads = _regs(ops[1])
            writes = _regs(ops[0])
            ws, j = 0, i - 1
            while j >= 0 and ws < max(MFMA_TO_VALU_DEFAULT, MFMA_SRC_TO_VALU_WRITE):
                pop, pops = _operands(ins[j])
                if pop.startswith("v_mfma") and pops:
                    dst = _regs(pops[0])
                    srcs = set().union(*[_regs(o) for o in pops[1:4]]) if len(pops) >= 4 else set()
                    if ws < _mfma_to_valu(pop) and dst & (reads | writes):
                        what = "reads" if dst & reads else "overwrites"
                        bad.append(f"{name}: MFMA {ins[j]!r} -> VALU {line!r} {what} its result after {ws} wait states")
                        break
                    if ws < MFMA_SRC_TO_VALU_WRITE and "f8f6f4" in pop and srcs & writes:
                        bad.append(f"{name}: MFMA {ins[j]!r} -> VALU {line!r} overwrites a source after {ws} wait states")
                        break
                ws += _ws(ins[j])
                j -= 1
    return bad


def kernel_names(text: str):
    """Symbols of every kernel in a device assembly listing (.amdhsa_kernel)."""
    return re.findall(r"^\s*\.amdhsa_kernel\s+(\S+)", text, flags=re.M)


def check_asm(text: str, kernels=None):
    """Check the named kernels (default: every kernel of the listing) in a
    device assembly listing; returns violations."""
    lines = text.splitlines()
    bad = []
    if kernels is None:
        kernels = kernel_names(text)
        if not kernels:
            return ["no kernel found in the assembly"]
    for kname in kernels:
        start = None
        for i, l in enumerate(lines):
            head = l.split(";")[0].strip()
            if head == kname + ":":
                start = i
                break
        if start is None:
            bad.append(f"kernel {kname} not found in the assembly")
            continue
        end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
        bad += check_function(lines[start:end + 1], kname)
    return bad


if __name__ == "__main__":
    problems = check_asm(open(sys.argv[1]).read())
    print("\n".join(problems) if problems else "no wait-state violations")
    sys.exit(1 if problems else 0)
