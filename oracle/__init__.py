"""CPU oracle for the MXFP8 ragged weight-gradient grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``mxfp8_ragged_grouped_amd``) never imports it, and it imports nothing from the
product path: the two share no code.

The arithmetic lives in ``mxw_oracle.c`` (plain C, fp64, ascending-token
accumulation; see its header for the definition and the format readings).  This
module only marshals numpy arrays into it through ``ctypes`` and builds it with
``gcc`` when asked.

What the oracle computes (blog post "Ragged MXFP8 Weight Gradients: A FlyDSL
Grouped GEMM on MI355X", section 1; ROCm blog "Group-GEMM in XLA", section
"Contracting"):

    dW[g][n][k] = sum_{m in [start_g, end_g)} e4m3(A[n][m]) 2^(sA[n][m/32]-127)
                                             * e4m3(B[k][m]) 2^(sB[k][m/32]-127)

It also holds the row-ragged grouped GEMM of the same layer (forward and data
gradient; blog section 1, XLA blog "non-contracting" ragged dot):

    out[m][n] = sum_{c < C} e4m3(X[m][c]) 2^(sX[m][c/32]-127)
                          * e4m3(W[g][n][c]) 2^(sW[g][n][c/32]-127),  m in [start_g, end_g)

the same weight gradient on plain bf16 operands (XLA blog, "Contracting"
ragged dot, Table 7's wgrad classes):

    dW[g][n][k] = sum_{m in [start_g, end_g)} bf16(A[n][m]) * bf16(B[k][m])

and the token-axis MXFP8 quantiser that produces the weight gradient's operands
(scale byte clamp(floor(log2 amax) - 8 + 127, 0, 254), E4M3 round-to-nearest-even
with saturation, transposed to token-contiguous).

Pins (all in ``tests/test_oracle_*.py``): every E4M3 and E8M0 code against the
format definition; a hand-computed two-expert case; exact rational brute force
on tiny random problems; the invariants (empty expert, scale-exponent doubling,
single expert = dense product, operand swap = transpose, expert split = sum,
padding garbage ignored); the XLA blog's small ragged-dot example in its
forward and weight-gradient forms; the XLA blog's group-lookup table.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxw_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libmxw_oracle.so")
_lib = None

ERRORS = {0: "ok", -1: "null pointer", -2: "bad dimension", -3: "malformed offs", -4: "out of memory"}


def build(force=True):
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no FP contraction)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.mxw_oracle_e4m3.restype = ctypes.c_double
    lib.mxw_oracle_e4m3.argtypes = [ctypes.c_uint]
    lib.mxw_oracle_e8m0.restype = ctypes.c_double
    lib.mxw_oracle_e8m0.argtypes = [ctypes.c_uint]
    lib.mxw_oracle_windows.argtypes = [P, I, I64, I, P, P]
    lib.mxw_oracle_ragged_contract_f64.argtypes = [P, P, P, P, I, I64, I, I, P]
    lib.mxw_oracle_decode_plane.argtypes = [P, P, I, I64, I64, P]
    lib.mxw_oracle_wgrad_f64.argtypes = [P, P, P, P, P, I, I64, I, I, P]
    lib.mxw_oracle_wgrad_points.argtypes = [P, P, P, P, P, I, I64, I, I, P, P, P, I64, P]
    lib.mxw_oracle_rows_contract_f64.argtypes = [P, P, P, P, I, I64, I, I, P]
    lib.mxw_oracle_rows_f64.argtypes = [P, P, P, P, P, I, I64, I, I, P]
    lib.mxw_oracle_rows_points.argtypes = [P, P, P, P, P, I, I64, I, I, P, P, I64, P]
    lib.mxw_oracle_quantize_tokens.argtypes = [P, I64, I, I64, P, P]
    lib.mxw_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.mxw_oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.mxw_oracle_to_bf16.argtypes = [P, I64, P]
    lib.mxw_oracle_bf16.restype = ctypes.c_double
    lib.mxw_oracle_bf16.argtypes = [ctypes.c_uint]
    lib.mxw_oracle_decode_bf16_plane.argtypes = [P, I, I64, I64, P]
    lib.mxw_oracle_bf16_wgrad_f64.argtypes = [P, P, P, I, I64, I, I, P]
    lib.mxw_oracle_bf16_wgrad_points.argtypes = [P, P, P, I, I64, I, I, P, P, P, I64, P]
    lib.mxw_oracle_max_threads.restype = I
    lib.mxw_oracle_set_threads.argtypes = [I]
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc):
    if rc != 0:
        raise ValueError("oracle error %d: %s" % (rc, ERRORS.get(rc, "?")))


def _u8(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a).view(np.uint8) if np.asarray(a).dtype != np.uint8 else np.asarray(a))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (shape, a.shape))
    return a


def e4m3(code):
    """Decode one OCP E4M3FN code to a Python float (NaN for S.1111.111)."""
    return _load().mxw_oracle_e4m3(int(code))


def e8m0(code):
    """Decode one E8M0 scale code: 2**(code-127); NaN for 0xFF."""
    return _load().mxw_oracle_e8m0(int(code))


def windows(offs, M, align=32):
    """(start, end) int64 arrays from the cumulative ends `offs`, validated:
    non-decreasing, <= M, multiples of `align` (32 for MXFP8 operands)."""
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    E = offs.shape[0]
    start = np.zeros(E, np.int64)
    end = np.zeros(E, np.int64)
    _check(_load().mxw_oracle_windows(_ptr(offs), E, int(M), int(align), _ptr(start), _ptr(end)))
    return start, end


def ragged_contract_f64(Ad, Bd, start, end):
    """Core contraction on decoded fp64 operands Ad [N,M], Bd [K,M] -> [E,N,K]."""
    Ad = np.ascontiguousarray(Ad, dtype=np.float64)
    Bd = np.ascontiguousarray(Bd, dtype=np.float64)
    start = np.ascontiguousarray(start, dtype=np.int64)
    end = np.ascontiguousarray(end, dtype=np.int64)
    N, M = Ad.shape
    K, M2 = Bd.shape
    if M2 != M or start.shape != end.shape:
        raise ValueError("shape mismatch")
    E = start.shape[0]
    out = np.empty((E, N, K), np.float64)
    _check(_load().mxw_oracle_ragged_contract_f64(_ptr(Ad), _ptr(Bd), _ptr(start), _ptr(end), E, M, N, K, _ptr(out)))
    return out


def decode_plane(q, s, used=None):
    """Decode an MXFP8 plane q [rows, M] (uint8 codes) with scales s [rows, M/32] to fp64."""
    q = _u8(q)
    rows, M = q.shape
    s = _u8(s, (rows, M // 32))
    used = M if used is None else int(used)
    out = np.empty((rows, M), np.float64)
    _check(_load().mxw_oracle_decode_plane(_ptr(q), _ptr(s), rows, M, used, _ptr(out)))
    return out


def wgrad_f64(A, sA, B, sB, offs):
    """Full fp64 weight gradient [E, N, K] of the MXFP8 operands."""
    A = _u8(A)
    N, M = A.shape
    B = _u8(B)
    K = B.shape[0]
    if B.shape[1] != M:
        raise ValueError("A and B disagree on M")
    sA = _u8(sA, (N, M // 32))
    sB = _u8(sB, (K, M // 32))
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    E = offs.shape[0]
    out = np.empty((E, N, K), np.float64)
    _check(_load().mxw_oracle_wgrad_f64(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(offs), E, M, N, K, _ptr(out)))
    return out


def wgrad_points(A, sA, B, sB, offs, g, n, k):
    """dW[g[i], n[i], k[i]] in fp64 for each i, straight from the definition."""
    A = _u8(A)
    N, M = A.shape
    B = _u8(B)
    K = B.shape[0]
    sA = _u8(sA, (N, M // 32))
    sB = _u8(sB, (K, M // 32))
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    g = np.ascontiguousarray(g, dtype=np.int32)
    n = np.ascontiguousarray(n, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.int32)
    if not (g.shape == n.shape == k.shape) or g.ndim != 1:
        raise ValueError("point index arrays must be 1-D and of equal length")
    out = np.empty(g.shape[0], np.float64)
    _check(_load().mxw_oracle_wgrad_points(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(offs), offs.shape[0], M, N, K,
                                           _ptr(g), _ptr(n), _ptr(k), g.shape[0], _ptr(out)))
    return out


def rows_contract_f64(Xd, Wd, start, end):
    """Row-ragged core on decoded fp64 operands Xd [M, C], Wd [E, Nw, C] ->
    [M, Nw]; rows outside every window are NaN."""
    Xd = np.ascontiguousarray(Xd, dtype=np.float64)
    Wd = np.ascontiguousarray(Wd, dtype=np.float64)
    start = np.ascontiguousarray(start, dtype=np.int64)
    end = np.ascontiguousarray(end, dtype=np.int64)
    M, C = Xd.shape
    E, Nw, C2 = Wd.shape
    if C2 != C or start.shape != (E,) or end.shape != (E,):
        raise ValueError("shape mismatch")
    out = np.full((M, Nw), np.nan)
    _check(_load().mxw_oracle_rows_contract_f64(_ptr(Xd), _ptr(Wd), _ptr(start), _ptr(end), E, M, C, Nw, _ptr(out)))
    return out


def rows_f64(X, sX, W, sW, offs):
    """Row-ragged grouped GEMM of MXFP8 operands X [M, C] (scales [M, C/32])
    and W [E, Nw, C] (scales [E, Nw, C/32]) -> fp64 [M, Nw]; rows past
    offs[E-1] are NaN (not part of any expert)."""
    X = _u8(X)
    M, C = X.shape
    W = _u8(W)
    E, Nw, C2 = W.shape
    if C2 != C:
        raise ValueError("X and W disagree on C")
    sX = _u8(sX, (M, C // 32))
    sW = _u8(sW, (E, Nw, C // 32))
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    if offs.shape != (E,):
        raise ValueError("offs must have one entry per expert")
    out = np.full((M, Nw), np.nan)
    _check(_load().mxw_oracle_rows_f64(_ptr(X), _ptr(sX), _ptr(W), _ptr(sW), _ptr(offs), E, M, C, Nw, _ptr(out)))
    return out


def rows_points(X, sX, W, sW, offs, m, n):
    """out[m[i], n[i]] of the row-ragged GEMM in fp64, straight from the
    definition (NaN for a row past the last expert)."""
    X = _u8(X)
    M, C = X.shape
    W = _u8(W)
    E, Nw, _ = W.shape
    sX = _u8(sX, (M, C // 32))
    sW = _u8(sW, (E, Nw, C // 32))
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int32)
    if m.shape != n.shape or m.ndim != 1:
        raise ValueError("point index arrays must be 1-D and of equal length")
    out = np.empty(m.shape[0], np.float64)
    _check(_load().mxw_oracle_rows_points(_ptr(X), _ptr(sX), _ptr(W), _ptr(sW), _ptr(offs), E, M, C, Nw, _ptr(m),
                                          _ptr(n), m.shape[0], _ptr(out)))
    return out


def quantize_tokens(x_bits, used=None):
    """Token-axis MXFP8 quantiser: bf16 bit patterns x [M, H] (uint16) ->
    (codes q [H, M], scales s [H, M/32]); tokens at or past `used` (default
    M) give code 0 and count as 0 in their block's amax."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M, H = x_bits.shape
    used = M if used is None else int(used)
    q = np.empty((H, M), np.uint8)
    s = np.empty((H, M // 32), np.uint8)
    _check(_load().mxw_oracle_quantize_tokens(_ptr(x_bits), M, H, used, _ptr(q), _ptr(s)))
    return q, s


def _u16(a):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        if a.dtype.itemsize != 2:
            raise ValueError("expected 16-bit bf16 bit patterns, got %s" % a.dtype)
        a = a.view(np.uint16)
    return np.ascontiguousarray(a)


def bf16(bits):
    """Decode one bf16 bit pattern to a Python float."""
    return _load().mxw_oracle_bf16(int(bits))


def decode_bf16_plane(x, used=None):
    """Decode a bf16 plane [rows, M] (uint16 bit patterns) to fp64; tokens at
    or past `used` are 0."""
    x = _u16(x)
    rows, M = x.shape
    used = M if used is None else int(used)
    out = np.empty((rows, M), np.float64)
    _check(_load().mxw_oracle_decode_bf16_plane(_ptr(x), rows, M, used, _ptr(out)))
    return out


def bf16_wgrad_f64(A, B, offs):
    """BF16 contracting ragged dot, fp64 [E, N, K]: A [N, M] and B [K, M] are
    bf16 bit patterns (uint16), token-contiguous; offs the cumulative ends
    (any alignment)."""
    A = _u16(A)
    B = _u16(B)
    N, M = A.shape
    K = B.shape[0]
    if B.shape[1] != M:
        raise ValueError("A and B disagree on M")
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    E = offs.shape[0]
    out = np.empty((E, N, K), np.float64)
    _check(_load().mxw_oracle_bf16_wgrad_f64(_ptr(A), _ptr(B), _ptr(offs), E, M, N, K, _ptr(out)))
    return out


def bf16_wgrad_points(A, B, offs, g, n, k):
    """BF16 dW[g[i], n[i], k[i]] in fp64 for each i, straight from the definition."""
    A = _u16(A)
    B = _u16(B)
    N, M = A.shape
    K = B.shape[0]
    if B.shape[1] != M:
        raise ValueError("A and B disagree on M")
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    g = np.ascontiguousarray(g, dtype=np.int32)
    n = np.ascontiguousarray(n, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.int32)
    if not (g.shape == n.shape == k.shape) or g.ndim != 1:
        raise ValueError("point index arrays must be 1-D and of equal length")
    out = np.empty(g.shape[0], np.float64)
    _check(_load().mxw_oracle_bf16_wgrad_points(_ptr(A), _ptr(B), _ptr(offs), offs.shape[0], M, N, K, _ptr(g),
                                                _ptr(n), _ptr(k), g.shape[0], _ptr(out)))
    return out


def to_bf16_bits(x):
    """Round fp64 values to bfloat16 bit patterns (uint16), nearest-even, in one step."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().mxw_oracle_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def max_threads():
    return _load().mxw_oracle_max_threads()


def set_threads(n):
    _load().mxw_oracle_set_threads(int(n))
