"""The C-ABI boundary on the CPU: the library loads, exports what include/hfa.h
declares, and rejects every invalid argument before making any HIP call.

Fake device addresses are used; they are never dereferenced because each call
here fails validation first.  The one call that passes validation (the
no-device case) runs only where no GPU is visible.
"""

import re
import subprocess
from pathlib import Path

import pytest
import torch

import fa2_fwd_amd as hfa

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "hfa.h"

GOOD = dict(q=0x100000, k=0x200000, v=0x300000, o=0x400000, lse=0x500000)


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hfa_[a-z_0-9]+)\s*\(", text)))


def _call(**kw):
    a = dict(GOOD, B=1, H=1, N=128, d=64, scale=0.125, dtype=hfa.HFA_F32, stream=None)
    a.update(kw)
    return hfa.hfa_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                            a["scale"], a["dtype"], a["stream"])


def test_library_exports_every_declared_symbol():
    lib = hfa.load_library()
    declared = _declared_functions()
    assert set(declared) == set(hfa.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", str(hfa.LIB_PATH)], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (hfa_\w+)", out))
    for name in declared:
        assert name in exported, f"{name} declared in hfa.h but not exported"
        assert getattr(lib, name) is not None


def test_library_is_gfx950_only(tmp_path):
    # The device code sits in the .hip_fatbin section; list its offload targets.
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fatbin}", str(hfa.LIB_PATH), str(tmp_path / "x.so")],
                   check=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o", f"--input={fatbin}"],
                         capture_output=True, text=True, check=True).stdout
    targets = [t for t in out.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets), out


def test_status_strings_distinct():
    codes = range(0, 10)
    strs = [hfa.hfa_status_str(c) for c in codes]
    assert len(set(strs)) == len(strs)
    assert hfa.hfa_status_str(99) == "unknown status"


def test_block_rows_table():
    for dt in (hfa.HFA_F32, hfa.HFA_BF16):
        for d in (64, 128):
            br = hfa.hfa_block_rows(dt, 1, 1, 1000, d)
            assert br > 0 and br % 16 == 0
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 1, 1000, 96) == 0
    assert hfa.hfa_block_rows(7, 1, 1, 1000, 64) == 0
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 0, 1, 1000, 128) == 0
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 1, 0, 128) == 0


def test_block_rows_follow_the_shape():
    # fp32 d=64 takes the tiling with the least rounds of workgroups (one per
    # CU, 256 CUs) times rows per workgroup over its relative throughput per
    # row (256 rows 1, 128 rows 0.86, 64 rows 0.6).
    assert hfa.hfa_block_rows(hfa.HFA_F32, 4, 8, 2048, 64) == 256  # one round of 256-row tiles
    assert hfa.hfa_block_rows(hfa.HFA_F32, 4, 8, 1024, 64) == 128  # one round of 128-row tiles
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 1, 128, 64) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 256, 200, 64) == 256
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 255, 256, 64) == 256
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 16, 1024, 64) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 8, 4096, 64) == 128
    # 384 workgroups of 256 rows (two rounds, the second half empty) against
    # 768 of 128 rows (three rounds): 128 rows
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 48, 2048, 64) == 128
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 80, 1024, 64) == 128
    # 192 workgroups of 256 rows (one round) against 384 of 128 (two): 256 rows
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 48, 1024, 64) == 256
    # one key tile or less: the shortest tile that still has the same rounds
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 256, 64, 64) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 256, 128, 64) == 128
    # bf16: 256-row ping-pong workgroups, or 128-row 4-wave ones for unsplit
    # calls whose 256-row grid has at most 128 workgroups (at d=128 only for
    # N <= 4096).
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 16, 16384, 128) == 256
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 2, 32, 4096, 128) == 256
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 16, 1024, 128) == 128
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 1, 128, 128) == 128
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 16, 2048, 128) == 128
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 1, 8192, 128) == 256
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 32, 2048, 128) == 256
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 4, 8, 1024, 64) == 128
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 1, 4, 4096, 64) == 128
    assert hfa.hfa_block_rows(hfa.HFA_BF16, 2, 16, 1536, 64) == 256
    # fp32 d=128 has two tilings: 128 rows when B*H*ceil(N/128) >= 256, else 64.
    assert hfa.hfa_block_rows(hfa.HFA_F32, 2, 8, 2048, 128) == 128
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 16, 2048, 128) == 128
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 16, 1024, 128) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 4, 4096, 128) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 255, 128, 128) == 64
    assert hfa.hfa_block_rows(hfa.HFA_F32, 1, 256, 100, 128) == 128


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), hfa.HFA_ERR_UNSUPPORTED),
    (dict(d=96), hfa.HFA_ERR_UNSUPPORTED),
    (dict(d=256), hfa.HFA_ERR_UNSUPPORTED),
    (dict(q=None), hfa.HFA_ERR_NULL),
    (dict(k=None), hfa.HFA_ERR_NULL),
    (dict(v=None), hfa.HFA_ERR_NULL),
    (dict(o=None), hfa.HFA_ERR_NULL),
    (dict(lse=None), hfa.HFA_ERR_NULL),
    (dict(B=0), hfa.HFA_ERR_SHAPE),
    (dict(H=0), hfa.HFA_ERR_SHAPE),
    (dict(N=0), hfa.HFA_ERR_SHAPE),
    (dict(N=-5), hfa.HFA_ERR_SHAPE),
    (dict(N=2**31 // 64 + 1), hfa.HFA_ERR_SHAPE),
    (dict(scale=float("nan")), hfa.HFA_ERR_SCALE),
    (dict(scale=float("inf")), hfa.HFA_ERR_SCALE),
    (dict(scale=float("-inf")), hfa.HFA_ERR_SCALE),
    (dict(q=0x100008), hfa.HFA_ERR_ALIGN),
    (dict(v=0x300004), hfa.HFA_ERR_ALIGN),
    (dict(o=0x400002), hfa.HFA_ERR_ALIGN),
    (dict(lse=0x500002), hfa.HFA_ERR_ALIGN),
    (dict(o=0x100000 + 64), hfa.HFA_ERR_ALIAS),          # o overlaps q
    (dict(lse=0x300000 + 16), hfa.HFA_ERR_ALIAS),        # lse overlaps v
    (dict(lse=0x400000 + 1024), hfa.HFA_ERR_ALIAS),      # lse overlaps o
])
def test_validation_rejects_before_any_device_call(kw, status):
    assert _call(**kw) == status


def test_inputs_may_alias_each_other():
    # q, k and v are read-only and may share memory; this must pass validation
    # (it then stops at the device check on a GPU-less host).
    if torch.cuda.is_available():
        pytest.skip("would launch on a visible GPU with fake pointers")
    assert _call(k=GOOD["q"], v=GOOD["q"]) == hfa.HFA_ERR_NO_DEVICE


def test_no_device_reported():
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    for dt in (hfa.HFA_F32, hfa.HFA_BF16):
        for d in (64, 128):
            assert _call(dtype=dt, d=d) == hfa.HFA_ERR_NO_DEVICE


def test_python_binding_value_errors():
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        hfa.attn_fwd(q, q, q)  # host tensors
    with pytest.raises(ValueError):
        hfa.attn_fwd(q, q[:, :, :4], q)
    with pytest.raises(ValueError):
        hfa.attn_fwd(q.double(), q.double(), q.double())
    with pytest.raises(ValueError):
        hfa.attn_fwd(q[0], q[0], q[0])


def _graph_create(count=1, **kw):
    a = dict(GOOD, B=1, H=1, N=128, d=64, scale=0.125, dtype=hfa.HFA_F32)
    a.update(kw)
    return hfa.hfa_attn_fwd_graph_create(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                         a["d"], a["scale"], a["dtype"], count)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), hfa.HFA_ERR_UNSUPPORTED),
    (dict(dtype=5), hfa.HFA_ERR_UNSUPPORTED),
    (dict(q=None), hfa.HFA_ERR_NULL),
    (dict(N=0), hfa.HFA_ERR_SHAPE),
    (dict(scale=float("inf")), hfa.HFA_ERR_SCALE),
    (dict(o=0x400004), hfa.HFA_ERR_ALIGN),
    (dict(lse=0x100010), hfa.HFA_ERR_ALIAS),
    (dict(count=0), hfa.HFA_ERR_SHAPE),
    (dict(count=(1 << 20) + 1), hfa.HFA_ERR_SHAPE),
])
def test_graph_create_validates_like_attn_fwd(kw, status):
    count = kw.pop("count", 1)
    st, h = _graph_create(count=count, **kw)
    assert st == status and h is None


def test_graph_null_handles():
    lib = hfa.load_library()
    assert hfa.hfa_graph_launch(None, None) == hfa.HFA_ERR_NULL
    hfa.hfa_graph_destroy(None)  # ignored
    import ctypes
    assert lib.hfa_attn_fwd_graph_create(0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 1, 1, 128, 64,
                                         0.125, hfa.HFA_F32, 1, None) == hfa.HFA_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), hfa.HFA_ERR_NULL),
    (dict(y=None), hfa.HFA_ERR_NULL),
    (dict(rows=0), hfa.HFA_ERR_SHAPE),
    (dict(cols=0), hfa.HFA_ERR_SHAPE),
    (dict(rows=1 << 31), hfa.HFA_ERR_SHAPE),
    (dict(rows=1 << 30, cols=1 << 33), hfa.HFA_ERR_SHAPE),
    (dict(x=0x100002), hfa.HFA_ERR_ALIGN),
    (dict(y=0x900001), hfa.HFA_ERR_ALIGN),
    (dict(y=0x100000 + 64), hfa.HFA_ERR_ALIAS),
])
def test_softmax_rows_rejects_before_any_hip_call(kw, status):
    a = dict(x=0x100000, y=0x900000, rows=4, cols=1000, stream=None)
    a.update(kw)
    assert hfa.hfa_softmax_rows(a["x"], a["y"], a["rows"], a["cols"], a["stream"]) == status


RMS_GOOD = dict(x=0x100000, r=0x200000, w=0x300000, y=0x400000, s=0x500000, rows=4, cols=1000, eps=1e-6,
                dtype=hfa.HFA_F32, stream=None)


def _rms(**kw):
    a = dict(RMS_GOOD)
    a.update(kw)
    return hfa.hfa_rmsnorm(a["x"], a["r"], a["w"], a["y"], a["s"], a["rows"], a["cols"], a["eps"], a["dtype"],
                           a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), hfa.HFA_ERR_NULL),
    (dict(w=None), hfa.HFA_ERR_NULL),
    (dict(y=None), hfa.HFA_ERR_NULL),
    (dict(s=None), hfa.HFA_ERR_NULL),
    (dict(dtype=5), hfa.HFA_ERR_UNSUPPORTED),
    (dict(rows=0), hfa.HFA_ERR_SHAPE),
    (dict(cols=0), hfa.HFA_ERR_SHAPE),
    (dict(cols=65537), hfa.HFA_ERR_SHAPE),
    (dict(rows=1 << 31), hfa.HFA_ERR_SHAPE),
    (dict(eps=0.0), hfa.HFA_ERR_EPS),
    (dict(eps=-1e-6), hfa.HFA_ERR_EPS),
    (dict(eps=float("inf")), hfa.HFA_ERR_EPS),
    (dict(eps=float("nan")), hfa.HFA_ERR_EPS),
    (dict(x=0x100002), hfa.HFA_ERR_ALIGN),
    (dict(w=0x300001, dtype=hfa.HFA_BF16), hfa.HFA_ERR_ALIGN),
    (dict(s=0x500002), hfa.HFA_ERR_ALIGN),
    (dict(y=0x100000 + 4), hfa.HFA_ERR_ALIAS),
    (dict(y=0x200000 - 8), hfa.HFA_ERR_ALIAS),
    (dict(y=0x300000 - 16), hfa.HFA_ERR_ALIAS),
    (dict(s=0x300000 + 4), hfa.HFA_ERR_ALIAS),
    (dict(s=0x400000), hfa.HFA_ERR_ALIAS),
    (dict(s=0x400000 + 400), hfa.HFA_ERR_ALIAS),
])
def test_rmsnorm_rejects_before_any_hip_call(kw, status):
    assert _rms(**kw) == status


def test_rmsnorm_accepts_in_place_and_no_residual():
    if torch.cuda.is_available():
        pytest.skip("would launch on a visible GPU with fake pointers")
    ok = hfa.HFA_ERR_NO_DEVICE  # validation passed; no device here
    assert _rms(y=RMS_GOOD["x"]) == ok
    assert _rms(s=RMS_GOOD["x"]) == ok
    assert _rms(y=RMS_GOOD["r"], s=RMS_GOOD["x"]) == ok
    assert _rms(r=None, s=None) == ok
    assert _rms(r=None, s=0x300000) == ok  # residual_out is ignored without a residual
    assert _rms(x=0x100002, w=0x300002, y=0x400002, r=None, dtype=hfa.HFA_BF16) == ok
    assert _rms(cols=65536, rows=1) == ok


def test_rmsnorm_binding_value_errors():
    x = torch.zeros(4, 16)
    w = torch.ones(16)
    with pytest.raises(ValueError):
        hfa.rmsnorm(x, w)  # host tensors
    with pytest.raises(ValueError):
        hfa.rmsnorm(x, torch.ones(15))
    with pytest.raises(ValueError):
        hfa.rmsnorm(x.double(), w.double())


# ---- key split entry point ---------------------------------------------------

WS = 0x10000000


def _split_call(splits=4, workspace=WS, workspace_bytes=1 << 30, **kw):
    a = dict(GOOD, B=1, H=2, N=1000, d=128, scale=0.125, dtype=hfa.HFA_BF16, stream=None)
    a.update(kw)
    return hfa.hfa_attn_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                                  a["scale"], a["dtype"], splits, workspace, workspace_bytes, a["stream"])


def test_split_plan_and_workspace_size():
    # B*H*ceil(N/256) row tiles below 256 split their keys (bf16 only); the
    # workspace holds [splits][B*H][N][d] + [splits][B*H][N] fp32.
    # as many ranges as fit one round of 256 workgroups, each >= 32 key tiles
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 8, 4096, 128) == 2
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 2, 16384, 128) == 2
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 1, 16384, 128) == 4
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 1, 32768, 64) == 2
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 1, 65536, 64) == 1    # 256 row tiles
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 16, 1024, 128) == 1    # ranges would be too short
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 16, 16384, 128) == 1   # 1024 workgroups already
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 2, 32, 4096, 128) == 1
    assert hfa.hfa_key_splits(hfa.HFA_F32, 1, 8, 4096, 64) == 1
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 1, 1, 64, 128) == 1       # one key tile: nothing to split
    assert hfa.hfa_key_splits(hfa.HFA_BF16, 0, 1, 64, 128) == 0
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 8, 4096, 128, 0) == 2 * 8 * 4096 * 129 * 4
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 16, 1024, 128, 0) == 0
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 16, 1024, 128, 4) == 4 * 16 * 1024 * 129 * 4
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 16, 1024, 128, 1) == 0
    # 16 key tiles asked to split 5 ways: ranges of 4 tiles, so 4 ranges
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 1, 1024, 64, 5) == 4 * 1024 * 65 * 4
    # more ranges than key tiles: one range per tile
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 1, 200, 64, 32) == 4 * 200 * 65 * 4
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 1, 1000, 64, 2) == -1
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 1, 1000, 64, -1) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(splits=-1), hfa.HFA_ERR_SHAPE),
    (dict(dtype=hfa.HFA_F32, d=64, splits=2), hfa.HFA_ERR_UNSUPPORTED),
    (dict(workspace=None), hfa.HFA_ERR_NULL),
    (dict(workspace=WS + 8), hfa.HFA_ERR_ALIGN),
    (dict(workspace_bytes=4 * 2 * 1000 * 129 * 4 - 1), hfa.HFA_ERR_WORKSPACE),
    (dict(workspace=GOOD["q"] - 4096), hfa.HFA_ERR_ALIAS),     # overlaps q
    (dict(workspace=GOOD["lse"]), hfa.HFA_ERR_ALIAS),          # overlaps lse
    (dict(N=0), hfa.HFA_ERR_SHAPE),
    (dict(o=None), hfa.HFA_ERR_NULL),
])
def test_split_validation_rejects_before_any_device_call(kw, status):
    assert _split_call(**kw) == status


def test_f32_packed_workspace_size():
    # fp32 has no key split; its workspace holds K and V formatted once per call:
    # ceil(N/64) tiles of 57344 bytes per head at d=64 (K slice planes, exponents
    # and statistics padded to 32 KiB, then the 24 KiB of V pieces), ceil(N/32)
    # tiles of 49152 bytes at d=128.  splits=1 gives it in any case, splits=0 only
    # where at least 8 workgroups of a head share each key tile.
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 1, 1000, 64, 1) == 16 * 57344
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 2, 3, 100, 128, 1) == 6 * 4 * 49152
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 1, 1, 64, 1) == 57344
    # B*H=32, N=2048, d=64: 256-row workgroups, 8 per head -> packs
    assert hfa.hfa_block_rows(hfa.HFA_F32, 4, 8, 2048, 64) == 256
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 4, 8, 2048, 64, 0) == 32 * 32 * 57344
    # B*H=32, N=1024: 128-row workgroups, 8 per head, but only 16 key tiles -> no packing
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 4, 8, 1024, 64, 0) == 0
    # B*H=256, N=200: one workgroup per head -> no packing
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 256, 200, 64, 0) == 0
    # B*H=1024, N=4096: 256-row workgroups, 16 per head, 64 key tiles -> packs
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 4, 256, 4096, 64, 0) == 1024 * 64 * 57344
    # d=128 (128-row workgroups, 32-key tiles): N=1024 gives 8 per head and 32 key
    # tiles, N=896 gives 7
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 4, 1024, 128, 0) == 4 * 32 * 49152
    assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 1, 4, 896, 128, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(workspace=WS + 8), hfa.HFA_ERR_ALIGN),
    (dict(workspace_bytes=2 * 16 * 57344 - 1), hfa.HFA_ERR_WORKSPACE),
    (dict(workspace=GOOD["k"] + 4096), hfa.HFA_ERR_ALIAS),      # overlaps k
    (dict(workspace=GOOD["o"] - 2 * 16 * 57344 + 16), hfa.HFA_ERR_ALIAS),  # ends inside o
])
def test_f32_packed_validation(kw, status):
    # B=1 H=2 N=1000 d=64 fp32: 2 x 16 tiles of 57344 bytes
    assert _split_call(splits=1, dtype=hfa.HFA_F32, d=64, **kw) == status


def test_split_one_needs_no_workspace():
    if torch.cuda.is_available():
        pytest.skip("would launch on a visible GPU with fake pointers")
    assert _split_call(splits=1, workspace=None, workspace_bytes=0) == hfa.HFA_ERR_NO_DEVICE
    assert _split_call(splits=4, workspace_bytes=4 * 2 * 1000 * 129 * 4) == hfa.HFA_ERR_NO_DEVICE
    # fp32: no workspace runs hfa_attn_fwd's path, one of the packed size the packed path
    assert _split_call(splits=1, dtype=hfa.HFA_F32, d=64, workspace=None, workspace_bytes=0) == hfa.HFA_ERR_NO_DEVICE
    assert _split_call(splits=0, dtype=hfa.HFA_F32, d=64, workspace_bytes=2 * 16 * 57344) == hfa.HFA_ERR_NO_DEVICE


def test_noalloc_rejects_before_any_device_call():
    # validation and the 64 MiB scratch limit come before any HIP call
    # fake addresses far enough apart for 64 MiB tensors
    a = dict(q=0x10_0000_0000, k=0x20_0000_0000, v=0x30_0000_0000, o=0x40_0000_0000, lse=0x50_0000_0000,
             B=1, H=64, N=4096, d=128)
    call = lambda splits, **kw: hfa.hfa_attn_fwd_split_noalloc(  # noqa: E731
        kw.get("q", a["q"]), a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], 0.125,
        kw.get("dtype", hfa.HFA_BF16), splits, None)
    assert call(8) == hfa.HFA_ERR_WORKSPACE            # 8 x 64 x 4096 x 129 x 4 bytes > 64 MiB
    assert call(-1) == hfa.HFA_ERR_SHAPE
    assert call(2, dtype=hfa.HFA_F32) == hfa.HFA_ERR_UNSUPPORTED
    assert call(2, q=None) == hfa.HFA_ERR_NULL
