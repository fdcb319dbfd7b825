"""Build-level check of the gfx950 code: no inline-asm write lands in the
destination registers of an MFMA that is still in flight, or in the
accumulator input registers of an MFMA just issued.

The kernels pass the thread index through a one-instruction inline-asm move
(so that lane-dependent addresses are recomputed where they are used). The
compiler's hazard recognizer does not hold such a move back: if an MFMA
result register is never read, the register allocator may hand it to the
move at once, and the MFMA's late write then overwrites the thread index.
Every result register that an instruction reads first is protected (the
compiler waits before that read), so the check looks for inline-asm writes
into an MFMA's destination, within a window of issue slots, with no read of
those registers in between.

An MFMA also reads its accumulator input (the last operand) over its first
cycles after issue. The compiler spaces its own vector writes into those
registers at least four issue slots from the MFMA (the closest it places them
in these kernels), but does not space an inline-asm write; the register
allocator may hand the MFMA's last use of a register to the asm output at
once. A write there within four slots is flagged too.

No GPU is needed: hipcc compiles the sources to gfx950 assembly with the
library's own flags.
"""
import os
import re
import subprocess

import pytest

from linear_recurrent_sequence_fwd_amd import build as B

WINDOW = 20   # issue slots (s_nop n counts n + 1); far above an MFMA's result latency

# the sources with inline asm
SOURCES = ["mlstm_fused.hip", "slstm.hip"]


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[])v(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def unprotected_asm_writes(lines, window=WINDOW):
    """(line, distance, mfma) for every inline-asm write into the destination
    of a preceding MFMA, within `window` issue slots in straight-line code,
    with no read of those registers before it."""
    found = []
    for i, t in enumerate(lines):
        if not t.startswith("v_mfma"):
            continue
        dst = _regs(t.split(None, 1)[1].split(",")[0])
        in_asm, dist = False, 0
        for j in range(i + 1, len(lines)):
            u = lines[j]
            if u.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if u.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not u or u.startswith(";") or u.startswith(".") or u.endswith(":"):
                continue
            ops = u.split(None, 1)
            op = ops[0]
            if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
                break
            dist += int(ops[1], 0) + 1 if op == "s_nop" else 1
            if dist > window:
                break
            if len(ops) < 2 or op == "s_nop":
                continue
            parts = ops[1].split(",")
            writes = _regs(parts[0])
            reads = _regs(",".join(parts[1:]))
            if not op.startswith("v_"):
                reads |= writes   # stores and other non-vector-ALU ops read their first operand
            if reads & dst:
                break
            if writes & dst:
                if in_asm:
                    found.append((j + 1, dist, t))
                break
    return found


SRCC_WINDOW = 4   # issue slots after an MFMA in which its accumulator input is still read


def asm_writes_into_accumulator_input(lines, window=SRCC_WINDOW):
    """(line, distance, mfma) for every inline-asm write into the accumulator
    input registers of an MFMA (other than its own destination) within
    `window` issue slots after it, in straight-line code."""
    found = []
    for i, t in enumerate(lines):
        if not t.startswith("v_mfma"):
            continue
        parts = t.split(None, 1)[1].split(",")
        srcc = _regs(parts[-1]) - _regs(parts[0])
        if not srcc:
            continue
        in_asm, dist = False, 0
        for j in range(i + 1, len(lines)):
            u = lines[j]
            if u.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if u.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not u or u.startswith(";") or u.startswith(".") or u.endswith(":"):
                continue
            ops = u.split(None, 1)
            op = ops[0]
            if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
                break
            dist += int(ops[1], 0) + 1 if op == "s_nop" else 1
            if dist > window:
                break
            if in_asm and op.startswith("v_") and len(ops) > 1 and _regs(ops[1].split(",")[0]) & srcc:
                found.append((j + 1, dist, t))
                break
    return found


def test_scanner_finds_a_planted_hazard():
    lines = [
        "v_mfma_f32_16x16x32_bf16 v[74:77], v[78:81], v[70:73], 0",
        ";;#ASMSTART",
        "v_mov_b32 v77, v0",
        ";;#ASMEND",
        "v_add_f32_e32 v74, v74, v75",
    ]
    assert unprotected_asm_writes(lines) == [(3, 1, lines[0])]
    # read first: the compiler's wait before the read protects the later write
    safe = lines[:1] + ["v_add_f32_e32 v1, v77, v2"] + lines[1:]
    assert unprotected_asm_writes(safe) == []
    # an asm write into the accumulator input of the MFMA just issued
    acc = [
        "v_mfma_f32_16x16x32_bf16 v[90:93], v[118:121], v[90:93], v[94:97]",
        ";;#ASMSTART",
        "v_mov_b32 v94, v0",
        ";;#ASMEND",
    ]
    assert asm_writes_into_accumulator_input(acc) == [(3, 1, acc[0])]
    # the same write after a four-cycle wait is out of the window
    spaced = acc[:2] + ["s_nop 3"] + acc[2:]
    assert asm_writes_into_accumulator_input(spaced) == []


@pytest.mark.parametrize("src", SOURCES)
def test_no_inline_asm_write_into_an_mfma_in_flight(src, tmp_path):
    out = tmp_path / (src + ".s")
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE,
           os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l.strip() for l in out.read_text().splitlines()]
    found = unprotected_asm_writes(lines)
    assert not found, "\n".join(f"{src}.s:{ln}: {d} slots after {m}" for ln, d, m in found)
    found = asm_writes_into_accumulator_input(lines)
    assert not found, "\n".join(f"{src}.s:{ln}: into the accumulator input, {d} slots after {m}"
                                 for ln, d, m in found)
