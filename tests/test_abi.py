"""The C-ABI library: loads, exports every declared symbol, and rejects bad
arguments on the host (CPU only; no call here reaches a device)."""
import ctypes
import os
import re
import subprocess

import pytest

import mxfp8_ragged_grouped_amd as mxw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8_wgrad.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?!#)\s*[\w\s\*]*?\b([a-z]\w+)\s*\(", text, flags=re.M)))


def declared_macros():
    text = open(HEADER).read()
    return {m: int(v) for m, v in re.findall(r"#define\s+(MXW_\w+)\s+\(?(-?\d+)\)?", text)}


def test_library_built():
    assert os.path.exists(mxw.library_path()), "run __graft_entry__.build() first"


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"mxfp8_wgrad_grouped", "mxfp8_wgrad_grouped_ws", "mxfp8_wgrad_workspace_size",
                          "bf16_wgrad_grouped", "bf16_wgrad_grouped_ws", "bf16_wgrad_workspace_size",
                          "mxw_grid_size", "mxw_columns", "mxw_tail_split", "mxfp8_grouped_fwd",
                          "mxw_fwd_grid_size", "mxfp8_quantize_tokens", "mxw_strerror", "mxw_version"}
    lib = ctypes.CDLL(mxw.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mxw.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_grid_size():
    # one workgroup per (expert, 256 x 256 tile)
    assert mxw.grid_size(4, 128, 256) == 4
    assert mxw.grid_size(8, 1408, 2048) == 8 * 6 * 8
    assert mxw.grid_size(32, 4096, 7168) == 32 * 16 * 28
    assert mxw.grid_size(32, 7168, 2048) == 32 * 28 * 8
    assert mxw.grid_size(0, 128, 128) == 0
    assert mxw.grid_size(257, 128, 128) == 0


def test_strerror_and_version():
    codes = declared_macros()
    for name in ("MXW_OK", "MXW_ERR_NULL", "MXW_ERR_DIM", "MXW_ERR_ALIGN", "MXW_ERR_DEVICE", "MXW_ERR_LAUNCH",
                 "MXW_ERR_WORKSPACE", "MXW_ERR_SCRATCH"):
        assert name in codes
        assert mxw.strerror(codes[name])
    assert mxw.strerror(-99) == "unknown error"
    assert mxw.version() >= 100


# fake, never-dereferenced device addresses: the host checks run before any device access
P = 0x10000


@pytest.mark.parametrize("args,code", [
    ((0, P, P, P, P, 4, 512, 128, 256, P), -1),            # NULL A
    ((P, P, P, P, P, 4, 512, 128, 256, 0), -1),            # NULL out
    ((P, P, P, P, P, 0, 512, 128, 256, P), -2),            # E = 0
    ((P, P, P, P, P, 257, 512, 128, 256, P), -2),          # E too large
    ((P, P, P, P, P, 4, 500, 128, 256, P), -2),            # M % 32 != 0
    ((P, P, P, P, P, 4, -32, 128, 256, P), -2),            # M < 0
    ((P, P, P, P, P, 4, 512, 120, 256, P), -2),            # N % 16 != 0
    ((P, P, P, P, P, 4, 512, 128, 8, P), -2),              # K < 16
    ((P, P, P, P, P, 4, 16 * 1024 * 1024, 128, 256, P), -2),  # M beyond the supported range
    ((P + 8, P, P, P, P, 4, 512, 128, 256, P), -3),        # A misaligned
    ((P, P, P, P, P, 4, 512, 128, 256, P + 2), -3),        # out misaligned
    ((P, P + 2, P, P, P, 4, 512, 128, 256, P), -3),        # sA not 4-byte aligned
    ((P, P, P, P + 1, P, 4, 512, 128, 256, P), -3),        # sB not 4-byte aligned
])
def test_host_argument_checks(args, code):
    assert mxw.mxfp8_wgrad_grouped(*args) == code
    # the workspace variant runs the same checks first (any workspace)
    assert mxw.mxfp8_wgrad_grouped_ws(*args, P, 1 << 30) == code
    assert mxw.mxfp8_wgrad_grouped_ws(*args, 0, 0) == code


def test_workspace_size_host_checks():
    """Invalid sizes are rejected before any device query; valid ones need the
    device's CU count, so on a host without a gfx950 they report no device."""
    lib = mxw._load()
    assert lib.mxfp8_wgrad_workspace_size(0, 512, 0, 128, 256) == -2
    assert lib.mxfp8_wgrad_workspace_size(4, 500, 0, 128, 256) == -2
    assert lib.mxfp8_wgrad_workspace_size(4, 512, 0, 120, 256) == -2
    assert lib.mxfp8_wgrad_workspace_size(4, 512, 480, 128, 256) == -2   # ld < M
    assert lib.mxfp8_wgrad_workspace_size(4, 512, 528, 128, 256) == -2   # ld % 32 != 0
    assert lib.bf16_wgrad_workspace_size(4, 520, 128, 256) == -2
    import torch
    if not torch.cuda.is_available():
        assert lib.mxfp8_wgrad_workspace_size(8, 196608, 0, 1408, 2048) == -4
        assert lib.mxfp8_wgrad_workspace_size(8, 196608, 196608 + 128, 1408, 2048) == -4
        assert mxw.mxfp8_wgrad_grouped_ws(P, P, P, P, P, 4, 512, 128, 256, P, 0, 0, 0) == -4


@pytest.mark.parametrize("ld,code", [(480, -2), (528, -2), (16 * 1024 * 1024, -2)])
def test_row_stride_host_checks(ld, code):
    """A row stride below M, not a multiple of 32, or beyond the token range is
    rejected on the host by the workspace entries and the quantiser."""
    args = (P, P, P, P, P, 4, 512, 128, 256, P)
    assert mxw.mxfp8_wgrad_grouped_ws(*args, P, 1 << 30, 0, ld=ld) == code
    assert mxw.mxfp8_wgrad_grouped_noalloc(*args, 0, ld=ld) == code
    assert mxw.mxfp8_quantize_tokens(P, P, 4, 512, 128, P, P, 0, ld=ld) == code


@pytest.mark.parametrize("args,code", [
    ((0, P, P, 4, 512, 128, 256, P), -1),            # NULL A
    ((P, 0, P, 4, 512, 128, 256, P), -1),            # NULL B
    ((P, P, 0, 4, 512, 128, 256, P), -1),            # NULL offs
    ((P, P, P, 4, 512, 128, 256, 0), -1),            # NULL out
    ((P, P, P, 0, 512, 128, 256, P), -2),            # E = 0
    ((P, P, P, 257, 512, 128, 256, P), -2),          # E too large
    ((P, P, P, 4, 520, 128, 256, P), -2),            # M % 16 != 0
    ((P, P, P, 4, -16, 128, 256, P), -2),            # M < 0
    ((P, P, P, 4, 512, 136, 256, P), -2),            # N % 16 != 0
    ((P, P, P, 4, 512, 128, 0, P), -2),              # K < 16
    ((P, P, P, 4, 4 * 1024 * 1024 + 16, 128, 256, P), -2),  # M beyond half the MXFP8 token range
    ((P + 2, P, P, 4, 512, 128, 256, P), -3),        # A misaligned
    ((P, P + 8, P, 4, 512, 128, 256, P), -3),        # B misaligned
    ((P, P, P, 4, 512, 128, 256, P + 4), -3),        # out misaligned
])
def test_bf16_host_argument_checks(args, code):
    assert mxw.bf16_wgrad_grouped(*args) == code
    assert mxw.bf16_wgrad_grouped_ws(*args, P, 1 << 30) == code


def test_bf16_python_face_validates():
    import torch
    A = torch.zeros((128, 512), dtype=torch.bfloat16)
    B = torch.zeros((256, 512), dtype=torch.bfloat16)
    offs = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(TypeError):
        mxw.wgrad_bf16(A.float(), B, offs)            # not bf16
    with pytest.raises(ValueError):
        mxw.wgrad_bf16(A, B[:, :256].contiguous(), offs)  # M mismatch
    with pytest.raises(ValueError):
        mxw.wgrad_bf16(A, B, offs)                    # CPU tensors are refused: no host fallback


def test_python_face_validates_shapes():
    import torch
    A = torch.zeros((128, 512), dtype=torch.uint8)
    sA = torch.zeros((128, 16), dtype=torch.uint8)
    B = torch.zeros((256, 512), dtype=torch.uint8)
    sB = torch.zeros((256, 15), dtype=torch.uint8)
    offs = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        mxw.wgrad(A, sA, B, sB, offs)          # sB has the wrong shape
    sB = torch.zeros((256, 16), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mxw.wgrad(A, sA, B, sB, offs)          # CPU tensors are refused: no host fallback
    with pytest.raises(TypeError):
        mxw.wgrad(A, sA, B, sB, offs.to(torch.int64))


def test_scale_shuffle_rule():
    """The pre-shuffle runs at long experts (M >= 4096 E) or unaligned scale
    rows (M % 512 != 0); host-only, no device needed."""
    assert mxw.scale_shuffle(8, 196608) and mxw.scale_shuffle(32, 262144)
    assert not mxw.scale_shuffle(8, 8192)          # 1,024 tokens per expert, aligned rows
    assert not mxw.scale_shuffle(8, 8192 + 32)     # short experts: direct loads, whatever the row alignment
    assert not mxw.scale_shuffle(8, 8192 + 128)
    assert mxw.scale_shuffle(2, 8192 + 32)         # long experts: shuffled, whatever the row alignment
    assert mxw.scale_shuffle(1, 4096) and not mxw.scale_shuffle(2, 4096)
    with pytest.raises(mxw.MxwError):
        mxw.scale_shuffle(0, 512)
    with pytest.raises(mxw.MxwError):
        mxw.scale_shuffle(4, 500)


def test_columns_host_checks():
    """mxw_columns rejects invalid sizes on the host, before any device query."""
    lib = ctypes.CDLL(mxw.library_path())
    lib.mxw_columns.restype = ctypes.c_int
    lib.mxw_columns.argtypes = [ctypes.c_int] * 4
    assert lib.mxw_columns(0, 8192, 256, 256) == -2
    assert lib.mxw_columns(257, 8192, 256, 256) == -2
    assert lib.mxw_columns(4, -32, 256, 256) == -2
    assert lib.mxw_columns(4, 8192, 8, 256) == -2


def test_fwd_grid_size():
    # (R / 256 + E) row tiles at most, times the column tiles, rounded up to 8
    assert mxw.fwd_grid_size(4, 512, 128) == 8          # (2 + 4) * 1 -> 8
    assert mxw.fwd_grid_size(8, 196608, 1408) == (768 + 8) * 6
    assert mxw.fwd_grid_size(32, 262144, 7168) == (1024 + 32) * 28
    assert mxw.fwd_grid_size(1, 0, 256) == 8
    assert mxw.fwd_grid_size(0, 512, 128) == 0
    assert mxw.fwd_grid_size(4, -1, 128) == 0
    assert mxw.fwd_grid_size(4, 512, 8) == 0


@pytest.mark.parametrize("args,code", [
    ((0, P, P, P, P, 4, 512, 256, 128, P), -1),            # NULL A
    ((P, P, P, 0, P, 4, 512, 256, 128, P), -1),            # NULL sB
    ((P, P, P, P, P, 0, 512, 256, 128, P), -2),            # E = 0
    ((P, P, P, P, P, 257, 512, 256, 128, P), -2),          # E too large
    ((P, P, P, P, P, 4, -1, 256, 128, P), -2),             # R < 0
    ((P, P, P, P, P, 4, 512, 48, 128, P), -2),             # C % 32 != 0
    ((P, P, P, P, P, 4, 512, 0, 128, P), -2),              # C = 0
    ((P, P, P, P, P, 4, 512, 256, 120, P), -2),            # N % 16 != 0
    ((P, P, P, P, P, 4, 512, 256, 131072, P), -2),         # N too large
    ((P, P, P + 8, P, P, 4, 512, 256, 128, P), -3),        # B misaligned
    ((P, P, P, P, P, 4, 512, 256, 128, P + 2), -3),        # out misaligned
    ((P, P + 1, P, P, P, 4, 512, 256, 128, P), -3),        # sA not 4-byte aligned
    ((P, P, P, P + 2, P, 4, 512, 256, 128, P), -3),        # sB not 4-byte aligned
])
def test_fwd_host_argument_checks(args, code):
    assert mxw.mxfp8_grouped_fwd(*args) == code


def test_fwd_python_face_validates_shapes():
    import torch
    A = torch.zeros((512, 256), dtype=torch.uint8)
    sA = torch.zeros((512, 8), dtype=torch.uint8)
    B = torch.zeros((4, 128, 256), dtype=torch.uint8)
    sB = torch.zeros((4, 128, 7), dtype=torch.uint8)
    offs = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        mxw.fwd(A, sA, B, sB, offs)            # sB has the wrong shape
    sB = torch.zeros((4, 128, 8), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mxw.fwd(A, sA, B, sB, offs[:3])        # one offs entry per expert
    with pytest.raises(ValueError):
        mxw.fwd(A, sA, B, sB, offs)            # CPU tensors are refused: no host fallback


@pytest.mark.parametrize("args,code", [
    ((0, P, 4, 512, 128, P, P), -1),               # NULL x
    ((P, P, 4, 512, 128, 0, P), -1),               # NULL q
    ((P, P, 4, 512, 128, P, 0), -1),               # NULL s
    ((P, P, 4, 500, 128, P, P), -2),               # M % 32 != 0
    ((P, P, 4, -32, 128, P, P), -2),               # M < 0
    ((P, P, 4, 512, 120, P, P), -2),               # H % 16 != 0
    ((P, P, 4, 512, 8, P, P), -2),                 # H < 16
    ((P, P, 0, 512, 128, P, P), -2),               # E = 0 with offs
    ((P, P, 300, 512, 128, P, P), -2),             # E too large
    ((P + 2, P, 4, 512, 128, P, P), -3),           # x misaligned
    ((P, P, 4, 512, 128, P + 8, P), -3),           # q misaligned
])
def test_quantize_host_argument_checks(args, code):
    assert mxw.mxfp8_quantize_tokens(*args) == code


def test_quantize_python_face_validates():
    import torch
    with pytest.raises(ValueError):
        mxw.quantize_tokens(torch.zeros((64, 32), dtype=torch.float32))   # not bf16
    with pytest.raises(ValueError):
        mxw.quantize_tokens(torch.zeros((64, 32), dtype=torch.bfloat16))  # CPU tensor: no host fallback
