"""Builds ``libhfa.so`` (the gfx950 attention library) in-tree with hipcc.

The library is built from every ``csrc/*.hip`` translation unit (one per
operation: attention, row softmax, ...), compiled for gfx950 only.  Packed-fp32 VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
LIB_PATH = PKG / "libhfa.so"
SOURCES = sorted((PKG / "csrc").glob("*.hip"))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # NaN inputs are outside the contract: min/max need no NaN canonicalisation.
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Wall",
    "-Wno-unused-result",
]


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: Path | None = None) -> Path:
    out = Path(out) if out is not None else LIB_PATH
    tmp = out.with_name(out.name + ".tmp")
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", str(ROOT / "include"),
           *(str(s) for s in SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    tmp.replace(out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
