"""Builds ``libhfa.so`` (the gfx950 attention library) in-tree with hipcc.

The library is built from every ``csrc/*.hip`` translation unit (one per
operation: attention, row softmax, ...), compiled for gfx950 only.

Each translation unit is compiled in two passes, the way hipcc itself does it
internally: a device pass that produces the gfx950 offload bundle, and a host
pass that embeds that bundle (``-fcuda-include-gpubinary``).  Splitting them
lets the device-only flags reach the device compiler alone: packed-fp32 VALU
instructions are disabled for all device code, and the host compiler, which
has no such feature, never sees the flag.  The host objects are then linked
into the shared library.  Translation units build in parallel.

``HFA_SANITIZE=1`` adds AddressSanitizer and UndefinedBehaviorSanitizer to
the host code only (argument validation and dispatch); device code is never
instrumented.
"""

from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
LIB_PATH = PKG / "libhfa.so"
SOURCES = sorted((PKG / "csrc").glob("*.hip"))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = ["--offload-arch=gfx950"]
COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    # NaN inputs are outside the contract: min/max need no NaN canonicalisation.
    "-fno-honor-nans",
    "-Wall",
    "-Wno-unused-result",
]
# Device pass only: no packed-fp32 VALU instructions in any kernel, and no
# IEEE-mode NaN quieting on min/max.
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mno-amdgpu-ieee"]
# -Xarch_host before each: the sanitizers reach host code only.
SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _sanitize() -> bool:
    return os.environ.get("HFA_SANITIZE", "") not in ("", "0")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _compile_tu(src: Path, workdir: Path, extra_flags: list[str], verbose: bool) -> Path:
    inc = ["-I", str(ROOT / "include")]
    fatbin = workdir / (src.stem + ".hipfb")
    obj = workdir / (src.stem + ".o")
    _run([HIPCC, *ARCH, *COMMON, *DEVICE_ONLY, *extra_flags, *inc, "--cuda-device-only", "-c", str(src),
          "-o", str(fatbin)], verbose)
    host_extra = SANITIZE if _sanitize() else []
    _run([HIPCC, *ARCH, *COMMON, *extra_flags, *host_extra, *inc, "--cuda-host-only", "-c", str(src),
          "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(fatbin), "-o", str(obj)], verbose)
    return obj


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: Path | None = None) -> Path:
    out = Path(out) if out is not None else LIB_PATH
    tmp = out.with_name(out.name + ".tmp")
    extra = list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="hfa_build_") as d:
        workdir = Path(d)
        with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as pool:
            objs = list(pool.map(lambda s: _compile_tu(s, workdir, extra, verbose), SOURCES))
        link_extra = SANITIZE if _sanitize() else []
        _run([HIPCC, *ARCH, "-shared", "-fPIC", *link_extra, *(str(o) for o in objs), "-o", str(tmp)], verbose)
    tmp.replace(out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
