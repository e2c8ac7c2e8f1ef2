"""Wait states around the kernels' inline assembly (CPU only: hipcc -S).

The compiler inserts the wait states that gfx950 needs between dependent
instructions it emits itself, but it cannot see into an inline-asm statement.
Each translation unit is compiled to gfx950 assembly with the library's own
device flags, and every instruction inside an inline-asm block is checked:

  * no VALU instruction at all (e.g. a hand-written v_readfirstlane: a VALU
    write of its source VGPR right before it needs one wait state, which the
    compiler then does not insert);
  * a load to LDS (global_load_lds_*) is not directly preceded by a scalar
    write of M0, which it reads (one wait state needed);
  * a vector-memory instruction reads no SGPR written by a VALU instruction
    (v_readfirstlane, v_cmp, ...) within the five wait states before it.

It also checks that thread and workgroup indices are read without calls (the
runtime's helpers are not inlined into kernels built without IEEE mode, and a
workgroup index returned by a call is no longer known to be uniform).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
from pathlib import Path

import pytest

from fa2_fwd_amd import build as B

VMEM = ("global_", "buffer_", "flat_", "scratch_")


def _assembly(src: Path, tmp: Path) -> list[str]:
    out = tmp / (src.stem + ".s")
    subprocess.run([B.HIPCC, *B.ARCH, *B.COMMON, *B.DEVICE_ONLY, "-I", str(B.ROOT / "include"),
                    "--cuda-device-only", "-S", str(src), "-o", str(out)], check=True, capture_output=True)
    return out.read_text().splitlines()


def _instructions(lines: list[str]):
    """(text, in_inline_asm, function) per instruction; labels as '<label>'."""
    inasm, fn = False, None
    for raw in lines:
        s = raw.strip()
        m = re.match(r"^(_Z\w+):", s)
        if m:
            fn = m.group(1)
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        if s.startswith(".LBB"):
            yield "<label>", False, fn
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        yield s.split(";")[0].strip(), inasm, fn


def _sgprs(text: str) -> set[int]:
    regs: set[int] = set()
    for m in re.finditer(r"s\[(\d+):(\d+)\]", text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", text):
        regs.add(int(m.group(1)))
    return regs


def _findings(lines: list[str]) -> list[str]:
    insts = list(_instructions(lines))
    found = []
    for i, (text, in_asm, fn) in enumerate(insts):
        if not in_asm:
            continue
        op = text.split()[0]
        if op.startswith("v_"):
            found.append(f"{fn}: VALU instruction in inline asm: {text}")
        if not op.startswith(VMEM):
            continue
        used = _sgprs(text[len(op):])
        waits = 0
        for j in range(i - 1, -1, -1):
            prev = insts[j][0]
            if prev == "<label>" or waits >= 5:
                break
            pop = prev.split()[0]
            dst = prev[len(pop):].split(",")[0]
            if pop.startswith("v_") and _sgprs(dst) & used:
                found.append(f"{fn}: {prev!r} then {text!r} after {waits} wait states")
            waits += int(prev.split()[1]) + 1 if pop == "s_nop" else 1
        if "_lds_" in op:
            prev = insts[i - 1][0]
            if prev.startswith("s_") and "m0" in prev.split(",")[0]:
                found.append(f"{fn}: {prev!r} directly before {text!r}")
    for raw in lines:
        if re.search(r"__ockl_get_(local|group)_id", raw):
            found.append(f"call to a work-item id helper: {raw.strip()}")
            break
    return found


@pytest.mark.slow
@pytest.mark.parametrize("src", B.SOURCES, ids=lambda p: p.name)
def test_inline_asm_wait_states(src, tmp_path):
    if not (os.path.exists(B.HIPCC) or shutil.which(B.HIPCC)):
        pytest.skip("hipcc not installed")
    found = _findings(_assembly(src, tmp_path))
    assert not found, "\n".join(found[:20])


def test_checker_flags_known_hazards():
    """The checker itself, on hand-made snippets of each hazard."""
    asm = [
        "_Zk:",
        "\tv_sub_u32_e32 v1, v3, v1",
        "\t;;#ASMSTART",
        "\tv_readfirstlane_b32 s2, v1",
        "\t;;#ASMEND",
        "\t;;#ASMSTART",
        "\ts_mov_b32 m0, s4",
        "\tglobal_load_lds_dwordx4 v2, s[6:7]",
        "\t;;#ASMEND",
        "\tv_readfirstlane_b32 s8, v5",
        "\ts_nop 1",
        "\t;;#ASMSTART",
        "\tglobal_load_dwordx4 v[8:11], v2, s[8:9]",
        "\t;;#ASMEND",
    ]
    found = _findings(asm)
    assert any("VALU instruction in inline asm" in f for f in found)
    assert any("directly before" in f for f in found)
    assert any("after 2 wait states" in f for f in found)
    clean = ["_Zk:", "\tv_readfirstlane_b32 s8, v5", "\ts_nop 4", "\t;;#ASMSTART",
             "\ts_mov_b32 m0, s4", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v2, s[8:9]", "\t;;#ASMEND"]
    assert _findings(clean) == []
