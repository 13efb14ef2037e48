"""CPU oracle for the half-precision GEMM path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of ``bench.py`` load
this package.  The product library never imports or links it, and it shares no
code with the GPU path: the arithmetic lives in ``oracle.c`` (plain C, fp64),
built by ``build()`` below with gcc into ``liboracle.so`` next to this file.

What it computes (see the header of ``oracle.c`` for the passages it follows):

* ``gemm``       D = alpha*op(A)*op(B) + beta*C_in (+ bias), out = RNE(D) to the
                 16-bit type; optional per-row sum of squares of the written row,
                 or the RMS row scale followed by SwiGLU (B then holds gate|up), or
                 an activation (ReLU, SiLU, tanh-form GELU) or the interleaved-pair
                 rotary position embedding applied before the rounding.
* ``strassen``   the same product through 1 or 2 levels of the Strassen (1969) or
                 Winograd 2x2 block recursion, in fp64 (identity check).
* ``decode`` / ``encode``  exact 16-bit <-> fp64 conversions, RNE on encode.
* ``gemm_f8``    the 8-bit GEMM A B^T on E4M3 / E5M2 values with per-tensor scales
                 or E8M0 scales per block of 32 along K (MXFP8), same epilogue and
                 rounding as ``gemm``; ``decode_f8`` / ``decode_e8m0`` the formats.
* ``bilinear``   (oracle/bilinear.py) block schemes as coefficient tables (U, V, W):
                 Strassen (1969), Winograd's form and the rectangular <2,2,3;11>, their
                 Brent equations checked exactly, and the product through a scheme.
* ``gemm_dense`` / ``gemm_f8_dense``  the unrounded product of every row through
                 one fp64 library matmul (whole-output checks at full size), with
                 the magnitude |alpha||A||B| + |beta||C| that ``elementwise_bound``
                 turns into a per-element rounding-error bound.

Every function is pinned by ``tests/test_oracle_pins.py`` against hand-worked
products, exact integer identities, invariants and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import bilinear  # noqa: E402,F401  (block schemes; pure numpy)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
EPI_BIAS, EPI_ROWSUMSQ, EPI_RMS_SWIGLU, EPI_ACT, EPI_ROPE = 1, 2, 4, 8, 16
ACT_RELU, ACT_SILU, ACT_GELU_TANH = 1, 2, 3
S69, WINOGRAD = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # FGEMM_ORACLE_LIB: another build of the same source (the tests' sanitizer build)
    path = os.environ.get("FGEMM_ORACLE_LIB", "")
    if not path:
        if not os.path.exists(_LIB):
            build(force=False)
        path = _LIB
    lib = ctypes.CDLL(path)
    i64, u16p, f64p, i64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_decode.restype = ctypes.c_double
    lib.oracle_decode.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.oracle_encode.restype = ctypes.c_uint16
    lib.oracle_encode.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_decode_array.argtypes = [u16p, f64p, i64, ctypes.c_int]
    lib.oracle_encode_array.argtypes = [f64p, u16p, i64, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                u16p, i64, u16p, i64, ctypes.c_double, u16p, i64, ctypes.c_int,
                                ctypes.c_int, u16p, f64p, i64, ctypes.c_double, i64p, i64,
                                f64p, u16p, f64p, ctypes.c_int]
    lib.oracle_gemm_ex.restype = ctypes.c_int
    lib.oracle_gemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                   u16p, i64, u16p, i64, ctypes.c_double, u16p, i64, ctypes.c_int,
                                   ctypes.c_int, u16p, f64p, i64, ctypes.c_double, ctypes.c_int,
                                   i64p, i64, ctypes.c_double, i64p, i64, f64p, u16p, f64p,
                                   ctypes.c_int]
    lib.oracle_swiglu_bwd.restype = ctypes.c_int
    lib.oracle_swiglu_bwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                      u16p, i64, u16p, i64, ctypes.c_int, f64p, f64p, i64,
                                      ctypes.c_double, i64p, i64, f64p, u16p, f64p, ctypes.c_int]
    lib.oracle_rms_bwd.restype = ctypes.c_int
    lib.oracle_rms_bwd.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                   u16p, i64, u16p, i64, ctypes.c_int, f64p, f64p, f64p, i64,
                                   ctypes.c_double, i64p, i64, f64p, u16p, ctypes.c_int]
    lib.oracle_strassen.restype = ctypes.c_int
    lib.oracle_strassen.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, u16p, i64, u16p,
                                    i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, f64p]
    lib.oracle_strassen_f64.restype = ctypes.c_int
    lib.oracle_strassen_f64.argtypes = [i64, i64, i64, f64p, f64p, ctypes.c_int, ctypes.c_int, f64p]
    lib.oracle_naive_f64.argtypes = [i64, i64, i64, f64p, f64p, f64p]
    lib.oracle_s69_products.restype = ctypes.c_int
    lib.oracle_s69_products.argtypes = [i64, f64p, f64p, f64p]
    lib.oracle_decode_f8.restype = ctypes.c_double
    lib.oracle_decode_f8.argtypes = [ctypes.c_uint8, ctypes.c_int]
    lib.oracle_decode_e8m0.restype = ctypes.c_double
    lib.oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_f4.restype = ctypes.c_double
    lib.oracle_decode_f4.argtypes = [ctypes.c_uint8]
    lib.oracle_quantize_mx.restype = ctypes.c_int
    lib.oracle_quantize_mx.argtypes = [u16p, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, i64, ctypes.c_void_p, i64]
    u8p = ctypes.c_void_p
    lib.oracle_gemm_f8.restype = ctypes.c_int
    lib.oracle_gemm_f8.argtypes = [i64, i64, i64, ctypes.c_double, u8p, i64, ctypes.c_int, u8p,
                                   i64, ctypes.c_int, ctypes.c_double, ctypes.c_double, u8p, i64,
                                   u8p, i64, ctypes.c_double, u16p, i64, ctypes.c_int,
                                   ctypes.c_int, u16p, i64p, i64, f64p, u16p, f64p, ctypes.c_int]
    _lib = lib
    return lib


E4M3, E5M2 = 0, 1   # OCP 8-bit float formats (values); E8M0 is the MX block scale
E2M1 = 2            # OCP 4-bit float (two values a byte, unpack_f4's order)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("16-bit inputs are passed as their uint16 bit patterns")
    return a


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_decode_array(_ptr(bits), _ptr(out), bits.size, dtype)
    return out


def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encode_array(_ptr(x), _ptr(out), x.size, dtype)
    return out


def gemm(A, B, *, transA=False, transB=False, alpha=1.0, beta=0.0, C=None, dtype=BF16,
         epi=0, bias=None, rms_ss=None, rms_n=0, rms_eps=1e-6, act=0, rope_pos=None,
         rope_head_dim=0, rope_theta=10000.0, rows=None, threads=None):
    """Reference GEMM on 16-bit bit patterns.

    A is M x K (or K x M when transA), B is K x N (or N x K when transB), both
    uint16 row-major.  Returns (D, Q, ss) for the selected rows: D the unrounded
    fp64 result, Q its RNE 16-bit bits, ss the per-row sum of squares of the
    written row (ROWSUMSQ only, else None).  For EPI_RMS_SWIGLU, rms_ss holds
    the fp64 sums of squares of the selected rows.  EPI_ACT applies activation
    `act` (ACT_RELU, ACT_SILU, ACT_GELU_TANH) and EPI_ROPE the rotary embedding
    with positions rope_pos (one per row of the output, all M rows), head width
    rope_head_dim and base rope_theta, both to alpha*acc + beta*C + bias.
    """
    A, B = _u16(A), _u16(B)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    Kb = B.shape[1] if transB else B.shape[0]
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    Nout = N // 2 if epi & EPI_RMS_SWIGLU else N
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = rows.size
    if beta != 0.0:
        C = _u16(C)
        if C.shape[0] != M or C.shape[1] < Nout:
            raise ValueError("C_in shape")
    else:
        C = None
    if bias is not None:
        bias = _u16(bias)
    if epi & EPI_RMS_SWIGLU:
        rms_ss = np.ascontiguousarray(rms_ss, dtype=np.float64)
        if rms_ss.size != nrows:
            raise ValueError("rms_ss must hold one value per selected row")
    pos = None
    if epi & EPI_ROPE:
        pos = np.ascontiguousarray(np.asarray(rope_pos, dtype=np.int64)[rows])
    D = np.empty((nrows, Nout), dtype=np.float64)
    Q = np.empty((nrows, Nout), dtype=np.uint16)
    ss = np.empty(nrows, dtype=np.float64) if epi & EPI_ROWSUMSQ else None
    rc = _load().oracle_gemm_ex(int(transA), int(transB), M, N, K, float(alpha), _ptr(A),
                                A.shape[1], _ptr(B), B.shape[1], float(beta), _ptr(C),
                                0 if C is None else C.shape[1], dtype, epi, _ptr(bias),
                                _ptr(rms_ss), rms_n, float(rms_eps), int(act), _ptr(pos),
                                int(rope_head_dim), float(rope_theta), _ptr(rows), nrows, _ptr(D),
                                _ptr(Q), _ptr(ss), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return D, Q, ss


def swiglu_bwd(A, B, dO, *, rms_ss, rms_n, rms_eps=1e-6, alpha=1.0, transA=False,
               transB=False, dtype=BF16, rows=None, threads=None):
    """Backward of the RMS + SwiGLU epilogue with the row scale held fixed.

    op(B) has 2*Nout columns (gate | up); dO (M x Nout, 16-bit bits) is the incoming
    gradient and rms_ss the fp64 sums of squares of the selected rows.  Returns
    (D, Q): the gradient with respect to op(A)op(B) for the selected rows,
    unrounded and RNE 16-bit bits, both nrows x 2*Nout, and rgrad, the gradient
    with respect to each selected row's scale r_i.
    """
    A, B = _u16(A), _u16(B)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    d = np.ascontiguousarray(decode(_u16(dO)[rows], dtype), dtype=np.float64)
    rms_ss = np.ascontiguousarray(rms_ss, dtype=np.float64)
    if d.shape != (rows.size, N // 2) or rms_ss.size != rows.size:
        raise ValueError("dO or rms_ss shape")
    D = np.empty((rows.size, N), dtype=np.float64)
    Q = np.empty((rows.size, N), dtype=np.uint16)
    rg = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_swiglu_bwd(int(transA), int(transB), M, N, K, float(alpha), _ptr(A),
                                   A.shape[1], _ptr(B), B.shape[1], dtype, _ptr(d), _ptr(rms_ss),
                                   rms_n, float(rms_eps), _ptr(rows), rows.size, _ptr(D), _ptr(Q),
                                   _ptr(rg), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_swiglu_bwd rejected its arguments")
    return D, Q, rg


def rms_bwd(A, B, X, *, rms_ss, rgrad, rms_n, rms_eps=1e-6, alpha=1.0, transA=False,
            transB=False, dtype=BF16, rows=None, threads=None):
    """alpha*op(A)op(B) + c_i X with c_i = -r_i^3 rgrad_i / n: the gradient of the
    RMS-normalised layer's input X (M x N, 16-bit bits).  rms_ss and rgrad hold one
    fp64 value per selected row.  Returns (D, Q) for the selected rows."""
    A, B = _u16(A), _u16(B)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    x = np.ascontiguousarray(decode(_u16(X)[rows], dtype), dtype=np.float64)
    rms_ss = np.ascontiguousarray(rms_ss, dtype=np.float64)
    rgrad = np.ascontiguousarray(rgrad, dtype=np.float64)
    if x.shape != (rows.size, N) or rms_ss.size != rows.size or rgrad.size != rows.size:
        raise ValueError("X, rms_ss or rgrad shape")
    D = np.empty((rows.size, N), dtype=np.float64)
    Q = np.empty((rows.size, N), dtype=np.uint16)
    rc = _load().oracle_rms_bwd(int(transA), int(transB), M, N, K, float(alpha), _ptr(A),
                                A.shape[1], _ptr(B), B.shape[1], dtype, _ptr(x), _ptr(rms_ss),
                                _ptr(rgrad), rms_n, float(rms_eps), _ptr(rows), rows.size, _ptr(D),
                                _ptr(Q), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_rms_bwd rejected its arguments")
    return D, Q


def strassen(A, B, *, depth, variant, transA=False, transB=False, dtype=BF16):
    """fp64 product through `depth` levels of the 2x2 recursion (no epilogue)."""
    A, B = _u16(A), _u16(B)
    M = A.shape[1] if transA else A.shape[0]
    K = A.shape[0] if transA else A.shape[1]
    N = B.shape[0] if transB else B.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_strassen(int(transA), int(transB), M, N, K, _ptr(A), A.shape[1], _ptr(B),
                                 B.shape[1], dtype, depth, variant, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_strassen rejected its arguments")
    return out


def strassen_f64(A, B, *, depth, variant):
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N), dtype=np.float64)
    if _load().oracle_strassen_f64(M, N, K, _ptr(A), _ptr(B), depth, variant, _ptr(out)) != 0:
        raise ValueError("oracle_strassen_f64 rejected its arguments")
    return out


def naive_f64(A, B):
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    out = np.empty((A.shape[0], B.shape[1]), dtype=np.float64)
    _load().oracle_naive_f64(A.shape[0], B.shape[1], A.shape[1], _ptr(A), _ptr(B), _ptr(out))
    return out


def s69_products(A, B):
    """The seven Strassen (1969) block products M1..M7 of one level (n x n, n even)."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    n = A.shape[0]
    out = np.empty((7, n // 2, n // 2), dtype=np.float64)
    if _load().oracle_s69_products(n, _ptr(A), _ptr(B), _ptr(out)) != 0:
        raise ValueError("n must be even")
    return out


def rel_fro(x, ref) -> float:
    """Normwise relative error ||x - ref||_F / ||ref||_F, accumulated in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("8-bit inputs are passed as their uint8 bit patterns")
    return a


def decode_f8(bits: np.ndarray, fmt: int) -> np.ndarray:
    """Exact fp64 values of E4M3 or E5M2 bit patterns (OCP encodings)."""
    bits = _u8(bits)
    lib = _load()
    table = np.array([lib.oracle_decode_f8(c, fmt) for c in range(256)], dtype=np.float64)
    return table[bits]


def decode_f4(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 values of E2M1 codes (the low nibble of each uint8)."""
    codes = _u8(codes) & 15
    lib = _load()
    table = np.array([lib.oracle_decode_f4(c) for c in range(16)], dtype=np.float64)
    return table[codes]


def unpack_f4(packed: np.ndarray) -> np.ndarray:
    """Rows of packed 4-bit values (uint8, two a byte) -> one E2M1 code per value:
    value 2i is the low nibble of byte i, value 2i + 1 its high nibble."""
    packed = _u8(packed)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


def pack_f4(codes: np.ndarray) -> np.ndarray:
    """The inverse of unpack_f4 (an even number of codes a row)."""
    codes = _u8(codes) & 15
    return np.ascontiguousarray((codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8))


def decode_e8m0(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values 2^(e-127) of E8M0 scale bytes (255 is NaN)."""
    bits = _u8(bits)
    lib = _load()
    table = np.array([lib.oracle_decode_e8m0(c) for c in range(256)], dtype=np.float64)
    return table[bits]


def gemm_f8(A, B, *, fmt_a=E4M3, fmt_b=E4M3, scale_a=1.0, scale_b=1.0, mx_a=None, mx_b=None,
            alpha=1.0, beta=0.0, C=None, dtype=BF16, epi=0, bias=None, rows=None, threads=None):
    """Reference 8-bit GEMM: A (M x K) and B (N x K), uint8 bit patterns of E4M3 or
    E5M2, both K-contiguous (the product is A B^T).  Each value counts as s * q
    with s the per-tensor scale, or, when mx_a / mx_b are given (uint8 E8M0 arrays
    of shape [rows][K/32]), its block's scale.  Returns (D, Q, ss) for the selected
    rows as gemm() does; epilogues BIAS and ROWSUMSQ."""
    A, B = _u8(A), _u8(B)
    M, K = A.shape
    N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} vs {Kb}")
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = rows.size
    if beta != 0.0:
        C = _u16(C)
    else:
        C = None
    if bias is not None:
        bias = _u16(bias)
    mx_a = None if mx_a is None else _u8(mx_a)
    mx_b = None if mx_b is None else _u8(mx_b)
    D = np.empty((nrows, N), dtype=np.float64)
    Q = np.empty((nrows, N), dtype=np.uint16)
    ss = np.empty(nrows, dtype=np.float64) if epi & EPI_ROWSUMSQ else None
    rc = _load().oracle_gemm_f8(M, N, K, float(alpha), _ptr(A), A.shape[1], fmt_a, _ptr(B),
                                B.shape[1], fmt_b, float(scale_a), float(scale_b), _ptr(mx_a),
                                0 if mx_a is None else mx_a.shape[1], _ptr(mx_b),
                                0 if mx_b is None else mx_b.shape[1], float(beta), _ptr(C),
                                0 if C is None else C.shape[1], dtype, epi, _ptr(bias),
                                _ptr(rows), nrows, _ptr(D), _ptr(Q), _ptr(ss),
                                threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f8 rejected its arguments")
    return D, Q, ss


def gemm_mxf4(A, B, mx_a, mx_b, *, alpha=1.0, beta=0.0, C=None, dtype=BF16, epi=0, bias=None,
              rows=None, threads=None):
    """Reference MXFP4 GEMM: A (M x K/2) and B (N x K/2) uint8 rows of packed E2M1
    values (unpack_f4's order), both K-contiguous (the product is A B^T); each value
    counts as s * q with s the E8M0 scale of its block of 32 along K (mx_a, mx_b:
    uint8 arrays [rows][>= K/32]).  Returns (D, Q, ss) for the selected rows as
    gemm_f8 does; epilogues BIAS and ROWSUMSQ."""
    A, B = _u8(A), _u8(B)
    M, K = A.shape[0], 2 * A.shape[1]
    N = B.shape[0]
    if 2 * B.shape[1] != K:
        raise ValueError(f"inner dimensions differ: {K} vs {2 * B.shape[1]}")
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = rows.size
    C = _u16(C) if beta != 0.0 else None
    if bias is not None:
        bias = _u16(bias)
    mx_a, mx_b = _u8(mx_a), _u8(mx_b)
    D = np.empty((nrows, N), dtype=np.float64)
    Q = np.empty((nrows, N), dtype=np.uint16)
    ss = np.empty(nrows, dtype=np.float64) if epi & EPI_ROWSUMSQ else None
    rc = _load().oracle_gemm_f8(M, N, K, float(alpha), _ptr(A), A.shape[1], E2M1, _ptr(B),
                                B.shape[1], E2M1, 1.0, 1.0, _ptr(mx_a), mx_a.shape[1], _ptr(mx_b),
                                mx_b.shape[1], float(beta), _ptr(C),
                                0 if C is None else C.shape[1], dtype, epi, _ptr(bias),
                                _ptr(rows), nrows, _ptr(D), _ptr(Q), _ptr(ss),
                                threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_f8 rejected its arguments")
    return D, Q, ss


def quantize_mx(X, dtype, fmt, *, transpose=False):
    """MX quantization of a 16-bit matrix X (rows x cols bit patterns): blocks of 32
    values along each row, or, with transpose, along each column of X, i.e. along
    the rows of X^T.  Returns (Q, S): Q the codes of the quantized matrix (X or X^T:
    one byte a value, or E2M1 packed two a byte), S its E8M0 scales [rows][len/32]."""
    X = _u16(X)
    rows, cols = X.shape
    orows, olen = (cols, rows) if transpose else (rows, cols)
    width = olen // 2 if fmt == E2M1 else olen
    Q = np.zeros((orows, width), dtype=np.uint8)
    S = np.zeros((orows, olen // 32), dtype=np.uint8)
    rc = _load().oracle_quantize_mx(_ptr(X), rows, cols, cols, dtype, fmt, int(bool(transpose)),
                                    _ptr(Q), width, _ptr(S), max(olen // 32, 1))
    if rc != 0:
        raise ValueError("oracle_quantize_mx rejected its arguments")
    return Q, S


def dequantize_mx(Q, S, fmt):
    """The fp64 values s * q of quantize_mx's output."""
    codes = unpack_f4(Q) if fmt == E2M1 else _u8(Q)
    vals = decode_f4(codes) if fmt == E2M1 else decode_f8(codes, fmt)
    return vals * np.repeat(decode_e8m0(_u8(S)), 32, axis=1)[:, :vals.shape[1]]


def gemm_mxf4_dense(A, B, mx_a, mx_b, *, alpha=1.0):
    """``gemm_mxf4``'s unrounded alpha * sum_k (s q_a)(s q_b) for every row with one
    fp64 library matmul, and the bound magnitude S = |alpha| |A'| |B'|^T."""
    a = decode_f4(unpack_f4(A))
    b = decode_f4(unpack_f4(B))
    K = a.shape[1]
    a = a * np.repeat(decode_e8m0(_u8(mx_a)[:, :K // 32]), 32, axis=1)
    b = b * np.repeat(decode_e8m0(_u8(mx_b)[:, :K // 32]), 32, axis=1)
    D = alpha * (a @ b.T)
    S = abs(alpha) * (np.abs(a) @ np.abs(b).T)
    return D, S


# ------------------------------------------------------------ whole-output references
def gemm_dense(A, B, *, transA=False, transB=False, alpha=1.0, beta=0.0, C=None, dtype=BF16,
               bound=True):
    """The unrounded product D = alpha*op(A)op(B) + beta*C of ``gemm`` for every
    row, with one fp64 library matmul as the step that forms sum_k a_ik b_kj (its
    summation order differs from ascending k by fp64 roundings only, about
    K*2^-53 relative, far below any 16-bit tolerance).  Also returns
    S = |alpha| |op(A)| |op(B)| + |beta| |C|: every rounding-error bound of a
    floating-point evaluation of D scales with S element by element (None when
    bound=False).  Inputs are 16-bit bit patterns as for ``gemm``."""
    a = decode(_u16(A), dtype)
    b = decode(_u16(B), dtype)
    if transA:
        a = a.T
    if transB:
        b = b.T
    if a.shape[1] != b.shape[0]:
        raise ValueError(f"inner dimensions differ: {a.shape[1]} vs {b.shape[0]}")
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    D = alpha * (a @ b)
    S = abs(alpha) * (np.abs(a) @ np.abs(b)) if bound else None
    if beta != 0.0:
        c = decode(_u16(C), dtype)[:, :D.shape[1]]
        D += beta * c
        if bound:
            S += abs(beta) * np.abs(c)
    return D, S


def gemm_f8_dense(A, B, *, fmt_a=E4M3, fmt_b=E4M3, scale_a=1.0, scale_b=1.0, mx_a=None,
                  mx_b=None, alpha=1.0):
    """``gemm_f8``'s unrounded alpha * sum_k (s q_a)(s q_b) for every row (A M x K, B
    N x K, K-contiguous) with one fp64 library matmul, and the matching bound
    magnitude S = |alpha| |A'| |B'|^T of the scaled values A', B'."""
    M, K = _u8(A).shape
    a = decode_f8(A, fmt_a)
    b = decode_f8(B, fmt_b)
    if mx_a is not None:
        a = a * np.repeat(decode_e8m0(_u8(mx_a)[:, :K // 32]), 32, axis=1)
        b = b * np.repeat(decode_e8m0(_u8(mx_b)[:, :K // 32]), 32, axis=1)
    else:
        a = a * float(scale_a)
        b = b * float(scale_b)
    D = alpha * (a @ b.T)
    S = abs(alpha) * (np.abs(a) @ np.abs(b).T)
    return D, S


def elementwise_bound(D, S, K, dtype, acc_unit=2.0 ** -23):
    """Per-element bound on |RNE16(fl32(D)) - D| for a product evaluated with fp32
    accumulation: |fl32(D) - D| <= g S with g = n u / (1 - n u), n = K + 4 (the K
    products' sums and the alpha, beta*C steps; u = 2^-23 also covers truncating
    adds), then one rounding to the 16-bit type, relative unit u16 = 2^-8 (bf16) or
    2^-11 (fp16), plus half the fp16 subnormal spacing:
    bound = u16 |D| + (1 + u16) g S (+ 2^-25 for fp16)."""
    n = float(K + 4)
    g = n * acc_unit / (1.0 - n * acc_unit)
    u16 = 2.0 ** -8 if dtype == BF16 else 2.0 ** -11
    tiny = 0.0 if dtype == BF16 else 2.0 ** -25  # half the fp16 subnormal spacing
    return u16 * np.abs(D) + (1.0 + u16) * g * S + tiny


def rms_swiglu_terms(Y, W2, *, rms_ss, rms_n, rms_eps=1e-6, alpha=1.0, dtype=BF16):
    """``gemm``'s EPI_RMS_SWIGLU output for every row, unrounded: H = Y W2 through one
    fp64 library matmul (W2 holds the gate columns, then the up columns), the row
    scale r_i = 1 / sqrt(rms_ss_i / rms_n + rms_eps), g = alpha r_i H_gate,
    u = alpha r_i H_up, out = g / (1 + e^-g) * u.  Returns (out, H, d_gate, d_up)
    with the partial derivatives d out / d H_gate = alpha r silu'(g) u and
    d out / d H_up = alpha r silu(g): an error dH in the sums moves out by
    d_gate dH_gate + d_up dH_up to first order."""
    y = decode(_u16(Y), dtype)
    w = decode(_u16(W2), dtype)
    H = y @ w
    nout = H.shape[1] // 2
    r = 1.0 / np.sqrt(np.asarray(rms_ss, dtype=np.float64) / rms_n + rms_eps)
    ar = alpha * r[:, None]
    g = ar * H[:, :nout]
    u = ar * H[:, nout:]
    sig = 1.0 / (1.0 + np.exp(-g))
    out = g * sig * u
    d_gate = ar * sig * (1.0 + g * (1.0 - sig)) * u
    d_up = ar * g * sig
    return out, H, d_gate, d_up


def rms_swiglu_dense(Y, W2, *, rms_ss, rms_n, rms_eps=1e-6, alpha=1.0, dtype=BF16,
                     bound=False):
    """The EPI_RMS_SWIGLU output of ``rms_swiglu_terms``.  With bound=True also
    returns E = |d_gate| S_gate + |d_up| S_up with S = |Y| |W2|: an fp32
    evaluation whose sums H carry errors <= gamma S moves out by at most gamma E
    to first order."""
    out, _, d_gate, d_up = rms_swiglu_terms(Y, W2, rms_ss=rms_ss, rms_n=rms_n,
                                            rms_eps=rms_eps, alpha=alpha, dtype=dtype)
    if not bound:
        return out
    S = np.abs(decode(_u16(Y), dtype)) @ np.abs(decode(_u16(W2), dtype))
    nout = out.shape[1]
    return out, np.abs(d_gate) * S[:, :nout] + np.abs(d_up) * S[:, nout:]
