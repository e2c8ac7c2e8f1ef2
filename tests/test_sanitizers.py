"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds made for this test alone, in a temporary directory:
  * the oracle (``oracle/build.py`` with ``HFA_SANITIZE=1``: g++ with ASan and
    UBSan, any finding aborts), driven by the oracle pin tests;
  * ``libhfa.so`` with the sanitizers on its host code only (argument
    validation, dispatch; ``HFA_SANITIZE=1`` in ``fa2_fwd_amd/build.py``),
    driven by the C-ABI boundary tests, none of which reaches a device.
Each suite runs in a child process that preloads the matching sanitizer
runtime (g++'s for the oracle, clang's for the hipcc-built library) and loads
the sanitized build through ``HFA_REF_LIB`` / ``HFA_LIB``.  A sanitizer report
ends the child with a non-zero status.
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CLANG_ASAN = Path("/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so")


def _gcc_runtime(name: str) -> Path | None:
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return None
    path = Path(p.strip())
    return path if path.is_absolute() and path.exists() else None


def _run_suite(test_file: str, env_extra: dict[str, str]) -> None:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    proc = subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / test_file), "-x", "-q",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True)
    tail = "\n".join((proc.stdout + proc.stderr).splitlines()[-40:])
    assert proc.returncode == 0, f"{test_file} under the sanitizers failed:\n{tail}"
    assert "Sanitizer" not in proc.stderr, tail


@pytest.mark.slow
def test_oracle_under_sanitizers(tmp_path, monkeypatch):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("g++ sanitizer runtimes not installed")
    from oracle.build import build

    monkeypatch.setenv("HFA_SANITIZE", "1")
    lib = build(out=tmp_path / "libhfa_ref.so")
    _run_suite("test_oracle_pins.py", {"HFA_REF_LIB": str(lib), "HFA_SANITIZE": "1",
                                       "LD_PRELOAD": f"{asan}:{ubsan}"})


@pytest.mark.slow
def test_host_validation_under_sanitizers(tmp_path, monkeypatch):
    if not CLANG_ASAN.exists():
        pytest.skip("clang's ASan runtime not installed")
    from fa2_fwd_amd.build import build

    monkeypatch.setenv("HFA_SANITIZE", "1")
    lib = build(out=tmp_path / "libhfa.so")
    _run_suite("test_boundary.py", {"HFA_LIB": str(lib), "LD_PRELOAD": str(CLANG_ASAN)})
