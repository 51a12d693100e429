"""Wait states after matrix instructions in the compiled gfx950 code.

A vector instruction that reads the result registers of a matrix (MFMA)
instruction must issue a number of wait states after it; the hardware does
not interlock.  In straight-line code the compiler pads every such read of the
16x16 products used here with at least 8 wait states.  It was found to miss
one case: a read reached through a taken branch right after the matrix
instruction, which made the multi-token kernel's scores wrong and
nondeterministic.  This test compiles every source to assembly with the
library's own flags and walks every path (fall-through and branch targets)
from each matrix instruction, requiring 8 wait states before any non-matrix
read of its result, or a read of it as a matrix instruction's A or B operand.
(Chained accumulation through the C operand is left to the compiler.)
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_decode_pa_amd import build as B

REQUIRED = 8

_REG = re.compile(r"([va])(?:\[(\d+):(\d+)\]|(\d+))")
_STORE = ("global_store", "buffer_store", "flat_store", "ds_write", "ds_bpermute", "ds_permute")


def _regs(tok: str) -> set:
    m = _REG.fullmatch(tok.strip().split(" ")[0])
    if not m:
        return set()
    kind = m.group(1)
    if m.group(4) is not None:
        return {(kind, int(m.group(4)))}
    return {(kind, i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def _parse(line: str):
    line = line.split(";")[0].strip()
    if not line or line.startswith(".") or line.endswith(":"):
        return None
    parts = line.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def _reads(op: str, ops: list) -> set:
    if op.startswith("v_mfma"):
        return _regs(ops[1]) | _regs(ops[2]) if len(ops) >= 3 else set()
    srcs = ops if op.startswith(_STORE) else ops[1:]
    out = set()
    for o in srcs:
        out |= _regs(o)
    return out


def audit(asm: str, required: int = REQUIRED) -> list:
    """(matrix line, reading line, wait states) for every read that comes too
    early along some path."""
    lines = asm.split("\n")
    labels = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(\.L\w+):", line)
        if m:
            labels[m.group(1)] = i
    findings = []
    for i, line in enumerate(lines):
        p = _parse(line)
        if not p or not p[0].startswith("v_mfma"):
            continue
        dst = _regs(p[1][0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, ws = stack.pop()
            while j < len(lines) and ws < required:
                q = _parse(lines[j])
                if q is None:
                    j += 1
                    continue
                op, ops = q
                if op == "s_endpgm":
                    break
                if _reads(op, ops) & dst:
                    findings.append((i + 1, j + 1, ws))
                    break
                if op == "s_nop":
                    ws += int(ops[0], 0) + 1
                else:
                    ws += 1
                if op.startswith("s_cbranch") or op == "s_branch":
                    t = labels.get(ops[0]) if ops else None
                    if t is not None and (t, ws) not in seen:
                        seen.add((t, ws))
                        stack.append((t + 1, ws))
                    if op == "s_branch":
                        break
                j += 1
    return findings


def test_audit_flags_a_read_behind_a_taken_branch():
    asm = "\n".join([
        "k:",
        "\tv_mfma_f32_16x16x32_bf16 v[26:29], v[80:83], v[68:71], 0",
        "\ts_cbranch_scc1 .LBB0_5",
        "\ts_nop 7",
        "\tv_mul_f32_e32 v24, s26, v26",
        ".LBB0_5:",
        "\tv_mul_f32_e32 v24, s26, v27",
        "\ts_endpgm",
    ])
    assert [(f[1], f[2]) for f in audit(asm)] == [(7, 1)]


def test_audit_accepts_padded_straight_line_reads():
    asm = "\n".join([
        "k:",
        "\tv_mfma_f32_16x16x16_bf16 v[2:5], v[30:31], v[26:27], v[2:5]",
        "\tv_mfma_f32_16x16x16_bf16 v[6:9], v[32:33], v[26:27], v[6:9]",
        "\ts_nop 6",
        "\tv_mul_f32_e32 v2, v2, v28",
        "\ts_endpgm",
    ])
    assert audit(asm) == []
    # one wait state short
    assert audit(asm.replace("s_nop 6", "s_nop 5")) != []


@pytest.mark.skipif(shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("source", B.SOURCES)
def test_no_early_read_of_a_matrix_result(source, tmp_path):
    out = str(tmp_path / (source + ".s"))
    res = subprocess.run(B.device_asm_command(source, out), capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = open(out).read()
    found = audit(asm)
    lines = asm.split("\n")
    msg = "\n".join(f"line {a}: {lines[a - 1].strip()}  ->  line {b}: {lines[b - 1].strip()} "
                    f"after {w} wait states" for a, b, w in found[:10])
    assert not found, msg
