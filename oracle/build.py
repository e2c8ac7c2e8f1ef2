"""Builds the CPU oracle ``libhfa_ref.so`` with g++ (no HIP, no GPU headers).

Test infrastructure only.  ``-O2`` without fast-math and without FMA
contraction keeps the fp64 arithmetic strict IEEE in source order.
``HFA_SANITIZE=1`` adds AddressSanitizer and UndefinedBehaviorSanitizer (any
finding aborts); the process that loads such a build must preload g++'s
libasan and libubsan.
"""

from __future__ import annotations

import os
import subprocess
from pathlib import Path

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "hfa_ref.cpp"


def build(verbose: bool = False, src: Path | None = None, out: Path | None = None) -> Path:
    src = Path(src) if src is not None else SOURCE
    out = Path(out) if out is not None else _HERE / "libhfa_ref.so"
    tmp = out.with_suffix(".so.tmp")
    cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", str(src), "-o", str(tmp)]
    if os.environ.get("HFA_SANITIZE", "") not in ("", "0"):
        cmd[1:1] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    tmp.replace(out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
