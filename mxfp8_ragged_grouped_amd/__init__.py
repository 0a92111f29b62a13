"""MI355X-native MXFP8 ragged grouped GEMMs.

    out = wgrad(A, sA, B, sB, offs)        # bf16 [E, N, K]
    out = wgrad(..., plain=True)           # the entry point that takes no workspace
    out = wgrad_bf16(A, B, offs)           # bf16 [E, N, K] from bf16 operands
    out = fwd(A, sA, B, sB, offs)          # bf16 [R, N]
    q, s = quantize_tokens(x, offs)        # MXFP8 operand [H, M] from bf16 [M, H]

computes, for every expert g (blog "Ragged MXFP8 Weight Gradients: A FlyDSL
Grouped GEMM on MI355X", section 1),

    dW[g] = dY[g]^T X[g]   over expert g's tokens [offs[g-1], offs[g])

from MXFP8 operands A = dY^T [N, M] and B = X^T [K, M] (E4M3 codes, token axis
contiguous) with E8M0 scale planes sA [N, M/32] and sB [K, M/32]; and the
row-ragged GEMM of the same layer (forward and data gradient):

    out[m] = A[m] B[g]^T   for the rows m of expert g, contraction over C

from A [R, C] and B [E, N, C] (contraction innermost, 32-element E8M0 blocks
along it); the same weight gradient on plain bf16 operands A = dY^T [N, M],
B = X^T [K, M] (the XLA blog's "contracting" ragged dot); and the token-axis
quantiser that makes the weight gradient's
operands from bf16 activations / gradients.  Everything
runs in the HIP library ``lib/libmxfp8_wgrad.so`` (C ABI in
``include/mxfp8_wgrad.h``); this module only checks tensor metadata and passes
device pointers and the current stream.  There is no fallback: if the library
is missing, or the device is not a gfx950, calls raise.

The weight gradients have two entry points each.  mxfp8_wgrad_grouped (and
bf16_wgrad_grouped) touch no memory but their operands and output: one
workgroup per (expert, output tile).  The _ws variants take a caller-owned
workspace (sized by mxfp8_wgrad_workspace_size) for column mode and the
scale pre-shuffle.  wgrad() and wgrad_bf16() use the _ws variants unless
plain=True, taking the workspace from torch's caching allocator on the
stream the call runs on (or from `workspace`, a uint8 device tensor).
"""
import ctypes
import os

import torch

from .build import LIB as _LIB_PATH

__all__ = ["wgrad", "mxfp8_wgrad_grouped", "mxfp8_wgrad_grouped_ws", "mxfp8_wgrad_grouped_noalloc", "workspace_size", "wgrad_bf16",
           "bf16_wgrad_grouped", "bf16_wgrad_grouped_ws", "bf16_workspace_size", "grid_size", "columns",
           "scale_shuffle", "tail_split", "fwd", "mxfp8_grouped_fwd", "fwd_grid_size", "quantize_tokens", "mxfp8_quantize_tokens",
           "strerror", "version", "library_path", "MxwError"]

_lib = None


class MxwError(RuntimeError):
    pass


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MxwError("HIP library not built: %s (run python -m mxfp8_ragged_grouped_amd.build)" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.mxfp8_wgrad_grouped.restype = I
    lib.mxfp8_wgrad_grouped.argtypes = [P, P, P, P, P, I, I, I, I, P, P]
    S = ctypes.c_size_t
    lib.mxfp8_wgrad_grouped_ws.restype = I
    lib.mxfp8_wgrad_grouped_ws.argtypes = [P, P, P, P, P, I, I, I, I, I, P, P, S, P]
    lib.mxfp8_wgrad_grouped_noalloc.restype = I
    lib.mxfp8_wgrad_grouped_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, P, P]
    lib.mxfp8_wgrad_workspace_size.restype = ctypes.c_int64
    lib.mxfp8_wgrad_workspace_size.argtypes = [I, I, I, I, I]
    lib.bf16_wgrad_grouped.restype = I
    lib.bf16_wgrad_grouped.argtypes = [P, P, P, I, I, I, I, P, P]
    lib.bf16_wgrad_grouped_ws.restype = I
    lib.bf16_wgrad_grouped_ws.argtypes = [P, P, P, I, I, I, I, P, P, S, P]
    lib.bf16_wgrad_workspace_size.restype = ctypes.c_int64
    lib.bf16_wgrad_workspace_size.argtypes = [I, I, I, I]
    lib.mxw_grid_size.restype = ctypes.c_int64
    lib.mxw_grid_size.argtypes = [I, I, I]
    lib.mxw_strerror.restype = ctypes.c_char_p
    lib.mxw_strerror.argtypes = [I]
    lib.mxw_version.restype = I
    lib.mxw_version.argtypes = []
    lib.mxw_columns.restype = I
    lib.mxw_columns.argtypes = [I, I, I, I]
    lib.mxw_tail_split.restype = I
    lib.mxw_tail_split.argtypes = [I, I, I, I]
    lib.mxw_scale_shuffle.restype = I
    lib.mxw_scale_shuffle.argtypes = [I, I]
    lib.mxfp8_grouped_fwd.restype = I
    lib.mxfp8_grouped_fwd.argtypes = [P, P, P, P, P, I, I, I, I, P, P]
    lib.mxw_fwd_grid_size.restype = ctypes.c_int64
    lib.mxw_fwd_grid_size.argtypes = [I, I, I]
    lib.mxfp8_quantize_tokens.restype = I
    lib.mxfp8_quantize_tokens.argtypes = [P, P, I, I, I, I, P, P, P]
    _lib = lib
    return lib


def strerror(code):
    return _load().mxw_strerror(int(code)).decode()


def version():
    return _load().mxw_version()


def grid_size(E, N, K):
    return int(_load().mxw_grid_size(int(E), int(N), int(K)))


def columns(E, M, N, K):
    """Columns of a column-mode launch for this shape on the current device
    (0: one workgroup per tile).  Raises MxwError on a status code."""
    rc = _load().mxw_columns(int(E), int(M), int(N), int(K))
    if rc < 0:
        raise MxwError("mxw_columns failed: %s" % strerror(rc))
    return rc


def tail_split(E, M, N, K):
    """Output tiles an MXFP8 weight-gradient call without column mode or
    pre-shuffle runs as two half tiles (same bits) on the current device."""
    rc = _load().mxw_tail_split(int(E), int(M), int(N), int(K))
    if rc < 0:
        raise MxwError("mxw_tail_split failed: %s" % strerror(rc))
    return rc


def scale_shuffle(E, M):
    """True if an MXFP8 weight-gradient call of (E, M) runs the scale
    pre-shuffle kernel before the main kernel."""
    rc = _load().mxw_scale_shuffle(int(E), int(M))
    if rc < 0:
        raise MxwError("mxw_scale_shuffle failed: %s" % strerror(rc))
    return bool(rc)


def mxfp8_wgrad_grouped(A, sA, B, sB, offs, E, M, N, K, out, stream=0):
    """Raw C-ABI call on device addresses (ints).  Returns the status code."""
    lib = _load()
    return lib.mxfp8_wgrad_grouped(A, sA, B, sB, offs, int(E), int(M), int(N), int(K), out, stream)


def mxfp8_wgrad_grouped_ws(A, sA, B, sB, offs, E, M, N, K, out, workspace, workspace_bytes, stream=0, ld=0):
    """Raw C-ABI call on device addresses (ints); ld = row stride (0: M).
    Returns the status code."""
    lib = _load()
    return lib.mxfp8_wgrad_grouped_ws(A, sA, B, sB, offs, int(E), int(M), int(ld), int(N), int(K), out, workspace,
                                      int(workspace_bytes), stream)


def mxfp8_wgrad_grouped_noalloc(A, sA, B, sB, offs, E, M, N, K, out, stream=0, ld=0):
    """Raw C-ABI call on device addresses (ints): the workspace entry on the
    library's static scratch (no allocation); ld = row stride (0: M).
    Returns the status code."""
    lib = _load()
    return lib.mxfp8_wgrad_grouped_noalloc(A, sA, B, sB, offs, int(E), int(M), int(ld), int(N), int(K), out, stream)


def workspace_size(E, M, N, K, ld=0):
    """Bytes of workspace mxfp8_wgrad_grouped_ws needs for this shape (row
    stride ld, 0 = M) on the current device (0: none).  Raises MxwError on a
    status code."""
    rc = _load().mxfp8_wgrad_workspace_size(int(E), int(M), int(ld), int(N), int(K))
    if rc < 0:
        raise MxwError("mxfp8_wgrad_workspace_size failed: %s" % strerror(rc))
    return int(rc)


def bf16_workspace_size(E, M, N, K):
    """Bytes of workspace bf16_wgrad_grouped_ws needs (0: none)."""
    rc = _load().bf16_wgrad_workspace_size(int(E), int(M), int(N), int(K))
    if rc < 0:
        raise MxwError("bf16_wgrad_workspace_size failed: %s" % strerror(rc))
    return int(rc)


def _workspace(need, dev, stream, workspace):
    """(pointer, bytes, tensor): the caller's workspace, or a fresh one from
    torch's caching allocator on `stream` (stream-ordered reuse)."""
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the same GPU")
        nbytes = workspace.numel() * workspace.element_size()
        if nbytes < need:
            raise ValueError("workspace holds %d bytes, the call needs %d" % (nbytes, need))
        return workspace.data_ptr(), nbytes, workspace
    if need == 0:
        return 0, 0, None
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return ws.data_ptr(), need, ws


def _as_u8(t, name):
    if t.dtype == torch.uint8:
        return t
    if t.dtype == getattr(torch, "float8_e4m3fn", None) and name in ("A", "B"):
        return t.view(torch.uint8)
    raise TypeError("%s must be uint8 (or float8_e4m3fn for data), got %s" % (name, t.dtype))


def _row_stride(t, name):
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError("%s must be a 2-D tensor with unit column stride and rows at least a row apart" % name)
    return t.stride(0)


def wgrad(A, sA, B, sB, offs, out=None, stream=None, workspace=None, plain=False):
    """dW [E, N, K] bf16 from MXFP8 operands (see module docstring).

    A: [N, M] uint8/float8_e4m3fn, sA: [N, M/32] uint8, B: [K, M], sB: [K, M/32],
    offs: [E] int32 cumulative expert ends, all on one CUDA(HIP) device.  A and
    B may be row-strided views ([:, :M] of [rows, ld] buffers, the same ld for
    both, and sA, sB then with row stride ld / 32): the workspace entry reads
    that layout (see mxfp8_wgrad_grouped_ws); the other tensors are
    contiguous.  `out` (optional) is a contiguous bf16 [E, N, K] tensor that is
    fully overwritten.  Runs on `stream` (default: the current stream) and does
    not synchronise.  plain=True calls mxfp8_wgrad_grouped (no workspace);
    otherwise mxfp8_wgrad_grouped_ws with `workspace` (a contiguous device
    tensor of at least workspace_size() bytes) or one taken from torch's
    caching allocator on that stream.
    """
    A = _as_u8(A, "A")
    B = _as_u8(B, "B")
    sA = _as_u8(sA, "sA")
    sB = _as_u8(sB, "sB")
    if A.dim() != 2 or B.dim() != 2 or sA.dim() != 2 or sB.dim() != 2 or offs.dim() != 1:
        raise ValueError("A, sA, B, sB must be 2-D and offs 1-D")
    N, M = A.shape
    K = B.shape[0]
    E = offs.shape[0]
    if B.shape[1] != M or sA.shape != (N, M // 32) or sB.shape != (K, M // 32):
        raise ValueError("shape mismatch: A %s sA %s B %s sB %s" % (tuple(A.shape), tuple(sA.shape),
                                                                     tuple(B.shape), tuple(sB.shape)))
    if offs.dtype != torch.int32:
        raise TypeError("offs must be int32")
    dev = A.device
    for name, t in (("A", A), ("sA", sA), ("B", B), ("sB", sB), ("offs", offs)):
        if t.device != dev or dev.type != "cuda":
            raise ValueError("%s must be on the same GPU as A" % name)
    if not offs.is_contiguous():
        raise ValueError("offs must be contiguous")
    if M == 0:
        ld = 0  # no tokens: nothing is read, the stride is moot
    else:
        ld = _row_stride(A, "A")
        if _row_stride(B, "B") != ld or (ld % 32):
            raise ValueError("A and B must share one row stride, a multiple of 32 (got %d, %d)" % (ld, B.stride(0)))
        for name, t in (("sA", sA), ("sB", sB)):
            if _row_stride(t, name) != ld // 32:
                raise ValueError("%s rows must be ld / 32 = %d bytes apart" % (name, ld // 32))
    if plain and ld not in (0, M):
        raise ValueError("the entry point without a workspace takes contiguous operands (row stride M)")
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (E, N, K) or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bf16 [E, N, K] tensor on the same device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    # with no tokens no operand byte is read (every window is empty and the
    # kernel writes zeros), but torch gives empty tensors NULL addresses
    ptrs = [t.data_ptr() if M else out.data_ptr() for t in (A, sA, B, sB)]
    with torch.cuda.device(dev):
        if plain:
            rc = mxfp8_wgrad_grouped(*ptrs, offs.data_ptr(), E, M, N, K, out.data_ptr(), stream.cuda_stream)
        else:
            wp, wb, ws = _workspace(workspace_size(E, M, N, K, ld), dev, stream, workspace)
            rc = mxfp8_wgrad_grouped_ws(*ptrs, offs.data_ptr(), E, M, N, K, out.data_ptr(), wp, wb,
                                        stream.cuda_stream, ld=ld)
            del ws
    if rc != 0:
        raise MxwError("mxfp8_wgrad_grouped%s failed (%d): %s" % ("" if plain else "_ws", rc, strerror(rc)))
    return out


def bf16_wgrad_grouped(A, B, offs, E, M, N, K, out, stream=0):
    """Raw C-ABI call on device addresses (ints).  Returns the status code."""
    lib = _load()
    return lib.bf16_wgrad_grouped(A, B, offs, int(E), int(M), int(N), int(K), out, stream)


def bf16_wgrad_grouped_ws(A, B, offs, E, M, N, K, out, workspace, workspace_bytes, stream=0):
    """Raw C-ABI call on device addresses (ints).  Returns the status code."""
    lib = _load()
    return lib.bf16_wgrad_grouped_ws(A, B, offs, int(E), int(M), int(N), int(K), out, workspace,
                                     int(workspace_bytes), stream)


def wgrad_bf16(A, B, offs, out=None, stream=None, workspace=None, plain=False):
    """dW [E, N, K] bf16 from bf16 operands: dW[g] = A[:, win_g] B[:, win_g]^T.

    A: [N, M] and B: [K, M] bfloat16 (token axis contiguous), offs: [E] int32
    cumulative expert ends (multiples of 16), all contiguous on one GPU.
    `out` (optional) is a contiguous bf16 [E, N, K] tensor that is fully
    overwritten.  Runs on `stream` (default: the current stream) and does not
    synchronise.  plain / workspace: as for wgrad().
    """
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if A.dim() != 2 or B.dim() != 2 or offs.dim() != 1:
        raise ValueError("A, B must be 2-D and offs 1-D")
    N, M = A.shape
    K = B.shape[0]
    E = offs.shape[0]
    if B.shape[1] != M:
        raise ValueError("shape mismatch: A %s B %s" % (tuple(A.shape), tuple(B.shape)))
    if offs.dtype != torch.int32:
        raise TypeError("offs must be int32")
    dev = A.device
    for name, t in (("A", A), ("B", B), ("offs", offs)):
        if t.device != dev or dev.type != "cuda":
            raise ValueError("%s must be on the same GPU as A" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if out is None:
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (E, N, K) or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bf16 [E, N, K] tensor on the same device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        if plain:
            rc = bf16_wgrad_grouped(A.data_ptr(), B.data_ptr(), offs.data_ptr(), E, M, N, K, out.data_ptr(),
                                    stream.cuda_stream)
        else:
            wp, wb, ws = _workspace(bf16_workspace_size(E, M, N, K), dev, stream, workspace)
            rc = bf16_wgrad_grouped_ws(A.data_ptr(), B.data_ptr(), offs.data_ptr(), E, M, N, K, out.data_ptr(),
                                       wp, wb, stream.cuda_stream)
            del ws
    if rc != 0:
        raise MxwError("bf16_wgrad_grouped%s failed (%d): %s" % ("" if plain else "_ws", rc, strerror(rc)))
    return out


def fwd_grid_size(E, R, N):
    return int(_load().mxw_fwd_grid_size(int(E), int(R), int(N)))


def mxfp8_grouped_fwd(A, sA, B, sB, offs, E, R, C, N, out, stream=0):
    """Raw C-ABI call on device addresses (ints).  Returns the status code."""
    lib = _load()
    return lib.mxfp8_grouped_fwd(A, sA, B, sB, offs, int(E), int(R), int(C), int(N), out, stream)


def fwd(A, sA, B, sB, offs, out=None, stream=None):
    """Row-ragged grouped GEMM, bf16 [R, N]: out[m] = A[m] . B[g]^T for the
    rows m of expert g (forward: A = activations, B = weights; data gradient:
    A = output gradient, B = the weights quantized along the other axis).

    A: [R, C] uint8/float8_e4m3fn, sA: [R, C/32] uint8, B: [E, N, C],
    sB: [E, N, C/32], offs: [E] int32 cumulative row ends, all contiguous on
    one GPU.  Rows past offs[E-1] are not written (a new `out` leaves them
    uninitialised).  Runs on `stream` (default: the current stream) and does
    not synchronise.
    """
    A = _as_u8(A, "A")
    B = _as_u8(B, "B")
    sA = _as_u8(sA, "sA")
    sB = _as_u8(sB, "sB")
    if A.dim() != 2 or sA.dim() != 2 or B.dim() != 3 or sB.dim() != 3 or offs.dim() != 1:
        raise ValueError("A, sA must be 2-D, B, sB 3-D and offs 1-D")
    R, C = A.shape
    E, N, C2 = B.shape
    if C2 != C or sA.shape != (R, C // 32) or sB.shape != (E, N, C // 32) or offs.shape[0] != E:
        raise ValueError("shape mismatch: A %s sA %s B %s sB %s offs %s" % (
            tuple(A.shape), tuple(sA.shape), tuple(B.shape), tuple(sB.shape), tuple(offs.shape)))
    if offs.dtype != torch.int32:
        raise TypeError("offs must be int32")
    dev = A.device
    for name, t in (("A", A), ("sA", sA), ("B", B), ("sB", sB), ("offs", offs)):
        if t.device != dev or dev.type != "cuda":
            raise ValueError("%s must be on the same GPU as A" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (R, N) or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bf16 [R, N] tensor on the same device")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = mxfp8_grouped_fwd(A.data_ptr(), sA.data_ptr(), B.data_ptr(), sB.data_ptr(), offs.data_ptr(),
                               E, R, C, N, out.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise MxwError("mxfp8_grouped_fwd failed (%d): %s" % (rc, strerror(rc)))
    return out


def mxfp8_quantize_tokens(x, offs, E, M, H, q, s, stream=0, ld=0):
    """Raw C-ABI call on device addresses (ints; offs may be 0; ld = row stride
    of q, 0 for M).  Returns the status code."""
    return _load().mxfp8_quantize_tokens(x, offs, int(E), int(M), int(ld), int(H), q, s, stream)


def quantize_tokens(x, offs=None, q=None, s=None, stream=None, ld=None):
    """Token-axis MXFP8 quantisation of bf16 x [M, H] -> (codes uint8 [H, M],
    scales uint8 [H, M/32]), the weight gradient's operand layout.  Tokens at
    or past offs[-1] (all tokens are used when offs is None) become code 0.
    With ld (a multiple of 32, >= M) the codes and scales are written into
    [H, ld] and [H, ld/32] buffers and returned as their [:, :M] and
    [:, :M/32] views (the padded rows mxfp8_wgrad_grouped_ws reads best);
    the padding columns are not written.  Runs on `stream` (default: the
    current stream) and does not synchronise."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous 2-D bf16 tensor on the GPU")
    M, H = x.shape
    dev = x.device
    if offs is not None:
        if offs.dtype != torch.int32 or offs.dim() != 1 or offs.device != dev or not offs.is_contiguous():
            raise ValueError("offs must be a contiguous int32 vector on the same GPU")
    ld = M if ld is None else int(ld)
    if ld < M or ld % 32:
        raise ValueError("ld must be a multiple of 32 and at least M")
    if q is None:
        q = torch.empty((H, ld), dtype=torch.uint8, device=dev)[:, :M]
    if s is None:
        s = torch.empty((H, ld // 32), dtype=torch.uint8, device=dev)[:, :M // 32]
    if tuple(q.shape) != (H, M) or q.dtype != torch.uint8 or q.device != dev or (M and q.stride() != (ld, 1)):
        raise ValueError("q must be a uint8 [H, M] tensor with row stride ld on the same GPU")
    if tuple(s.shape) != (H, M // 32) or s.dtype != torch.uint8 or s.device != dev or (
            M and (s.stride(0) != ld // 32 or s.stride(1) != 1)):
        raise ValueError("s must be a uint8 [H, M/32] tensor with row stride ld / 32 on the same GPU")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = mxfp8_quantize_tokens(x.data_ptr(), 0 if offs is None else offs.data_ptr(),
                                   1 if offs is None else offs.shape[0], M, H, q.data_ptr(), s.data_ptr(),
                                   stream.cuda_stream, ld=ld)
    if rc != 0:
        raise MxwError("mxfp8_quantize_tokens failed (%d): %s" % (rc, strerror(rc)))
    return q, s
