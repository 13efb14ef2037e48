"""ctypes binding of libfgemm (include/fgemm.h) — argument marshalling only.

Every entry point of the C ABI has a function of the same name here.  All compute
runs in the library's HIP kernels; this module never computes results itself and
raises when the library is missing.  Torch tensors are accepted for convenience:
their device pointers, leading dimensions and the current HIP stream are passed
through unchanged.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfgemm.so")

# enums of fgemm.h
FGEMM_OK, FGEMM_ERR_INVALID_VALUE, FGEMM_ERR_NOT_SUPPORTED = 0, 1, 2
FGEMM_ERR_WORKSPACE, FGEMM_ERR_ALLOC, FGEMM_ERR_HIP = 3, 4, 5
FGEMM_OP_N, FGEMM_OP_T = 0, 1
FGEMM_F16, FGEMM_BF16 = 0, 1
FGEMM_EPI_NONE, FGEMM_EPI_BIAS, FGEMM_EPI_ROWSUMSQ, FGEMM_EPI_RMS_SWIGLU = 0, 1, 2, 4
FGEMM_EPI_ACT, FGEMM_EPI_ROPE, FGEMM_EPI_SWIGLU_BWD, FGEMM_EPI_RMS_BWD = 8, 16, 32, 64
FGEMM_ACT_RELU, FGEMM_ACT_SILU, FGEMM_ACT_GELU_TANH = 1, 2, 3
FGEMM_PATH_CLASSICAL, FGEMM_PATH_STRASSEN = 0, 1
FGEMM_VARIANT_S69, FGEMM_VARIANT_WINOGRAD, FGEMM_VARIANT_R223 = 0, 1, 2
FGEMM_E4M3, FGEMM_E5M2, FGEMM_E2M1 = 0, 1, 2

# every symbol include/fgemm.h declares
EXPORTS = ("fgemm_create", "fgemm_destroy", "fgemm_set_workspace", "fgemm_get_model",
           "fgemm_set_model", "fgemm_select", "fgemm_select_model", "fgemm_gemm",
           "fgemm_gemm_plan", "fgemm_gemm_noalloc", "fgemm_gemm_f8", "fgemm_gemm_mxf8",
           "fgemm_gemm_mxf4", "fgemm_quantize_mx",
           "fgemm_check_args",
           "fgemm_tile_count",
           "fgemm_wave_count", "fgemm_plan_rel_err", "fgemm_read_probe", "fgemm_status_string")

# FGEMM_NOALLOC_SCRATCH_BYTES and FGEMM_READ_PROBE_GROUPS of fgemm.h
FGEMM_NOALLOC_SCRATCH_BYTES = 64 << 20
FGEMM_READ_PROBE_GROUPS = 1024


class FgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_name(status)}")
        self.status = status


class fgemm_epilogue_t(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("bias", ctypes.c_void_p),
                ("rowsumsq", ctypes.c_void_p), ("rms_rowsumsq", ctypes.c_void_p),
                ("rms_n", ctypes.c_int64), ("rms_eps", ctypes.c_float),
                ("act", ctypes.c_int32), ("rope_positions", ctypes.c_void_p),
                ("rope_offset", ctypes.c_int64), ("rope_head_dim", ctypes.c_int64),
                ("rope_theta", ctypes.c_float), ("swiglu_dout", ctypes.c_void_p),
                ("swiglu_ldd", ctypes.c_int64), ("rms_grad", ctypes.c_void_p),
                ("rms_x", ctypes.c_void_p), ("rms_ldx", ctypes.c_int64)]


class fgemm_plan_t(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("depth", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("t_pred_us", ctypes.c_double),
                ("t_classical_pred_us", ctypes.c_double), ("pred_rel_err", ctypes.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class fgemm_model_t(ctypes.Structure):
    _fields_ = [("compute_units", ctypes.c_int32), ("peak_tflops", ctypes.c_double),
                ("hbm_gbps", ctypes.c_double), ("eta_mfma", ctypes.c_double),
                ("eta_hbm", ctypes.c_double), ("launch_us", ctypes.c_double),
                ("max_workspace_bytes", ctypes.c_double), ("max_rel_err", ctypes.c_double)]


_lib = None


def lib():
    """Load libfgemm.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m hgemm_strassen_type_amd.build` (no fallback exists)")
    # torch first: its HIP runtime and the system one share a soname, and whichever is
    # loaded first serves the process; handles are used with torch's device memory and
    # streams, so that must be torch's (loading the library first made fgemm_create
    # fail once torch initialised the GPU)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    st = ctypes.c_int
    epi_p = ctypes.POINTER(fgemm_epilogue_t)
    plan_p = ctypes.POINTER(fgemm_plan_t)
    model_p = ctypes.POINTER(fgemm_model_t)
    sig = {
        "fgemm_create": (st, [ctypes.POINTER(vp), i32]),
        "fgemm_destroy": (st, [vp]),
        "fgemm_set_workspace": (st, [vp, vp, ctypes.c_size_t]),
        "fgemm_get_model": (st, [vp, model_p]),
        "fgemm_set_model": (st, [vp, model_p]),
        "fgemm_select": (st, [vp, i32, i32, i64, i64, i64, i32, epi_p, plan_p]),
        "fgemm_select_model": (st, [model_p, i32, i32, i64, i64, i64, i32, epi_p, plan_p]),
        "fgemm_gemm": (st, [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64,
                            i32, epi_p, vp]),
        "fgemm_gemm_plan": (st, [vp, plan_p, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32,
                                 vp, i64, i32, epi_p, vp]),
        "fgemm_gemm_noalloc": (st, [vp, i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp,
                                    i64, i32, epi_p, vp]),
        "fgemm_gemm_f8": (st, [vp, i64, i64, i64, f32, vp, i64, i32, f32, vp, i64, i32, f32, f32,
                               vp, i64, i32, epi_p, vp]),
        "fgemm_gemm_mxf8": (st, [vp, i64, i64, i64, f32, vp, i64, i32, vp, i64, vp, i64, i32, vp,
                                 i64, f32, vp, i64, i32, epi_p, vp]),
        "fgemm_gemm_mxf4": (st, [vp, i64, i64, i64, f32, vp, i64, vp, i64, vp, i64, vp, i64, f32,
                                 vp, i64, i32, epi_p, vp]),
        "fgemm_quantize_mx": (st, [vp, i64, i64, i64, i32, i32, i32, vp, i64, vp, i64, vp]),
        "fgemm_check_args": (st, [i32, i32, i64, i64, i64, vp, i64, vp, i64, f32, vp, i64, i32,
                                  epi_p]),
        "fgemm_tile_count": (i64, [i64, i64, i64, i64]),
        "fgemm_wave_count": (i64, [i64, i64, ctypes.POINTER(ctypes.c_double)]),
        "fgemm_plan_rel_err": (ctypes.c_double, [i32, plan_p]),
        "fgemm_read_probe": (st, [vp, i64, vp, vp]),
        "fgemm_status_string": (ctypes.c_char_p, [st]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_name(status: int) -> str:
    return lib().fgemm_status_string(status).decode()


def _check(status: int, where: str):
    if status != FGEMM_OK:
        raise FgemmError(status, where)


# ------------------------------------------------------------------ raw ABI calls
def fgemm_create(device: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(lib().fgemm_create(ctypes.byref(h), device), "fgemm_create")
    return h.value


def fgemm_destroy(handle: int):
    _check(lib().fgemm_destroy(handle), "fgemm_destroy")


def fgemm_set_workspace(handle: int, dptr: int, nbytes: int):
    _check(lib().fgemm_set_workspace(handle, dptr, nbytes), "fgemm_set_workspace")


def fgemm_get_model(handle: int) -> fgemm_model_t:
    m = fgemm_model_t()
    _check(lib().fgemm_get_model(handle, ctypes.byref(m)), "fgemm_get_model")
    return m


def fgemm_set_model(handle: int, model: fgemm_model_t):
    _check(lib().fgemm_set_model(handle, ctypes.byref(model)), "fgemm_set_model")


def make_epilogue(flags=0, bias=0, rowsumsq=0, rms_rowsumsq=0, rms_n=0, rms_eps=0.0, act=0,
                  rope_positions=0, rope_offset=0, rope_head_dim=0, rope_theta=10000.0,
                  swiglu_dout=0, swiglu_ldd=0, rms_grad=0, rms_x=0, rms_ldx=0):
    return fgemm_epilogue_t(flags, bias or None, rowsumsq or None, rms_rowsumsq or None, rms_n,
                            rms_eps, act, rope_positions or None, rope_offset, rope_head_dim,
                            rope_theta, swiglu_dout or None, swiglu_ldd, rms_grad or None,
                            rms_x or None, rms_ldx)


def fgemm_select(handle, transA, transB, M, N, K, dtype, epilogue=None) -> fgemm_plan_t:
    p = fgemm_plan_t()
    e = ctypes.byref(epilogue) if epilogue is not None else None
    _check(lib().fgemm_select(handle, transA, transB, M, N, K, dtype, e, ctypes.byref(p)),
           "fgemm_select")
    return p


def fgemm_select_model(model, transA, transB, M, N, K, dtype, epilogue=None) -> fgemm_plan_t:
    p = fgemm_plan_t()
    e = ctypes.byref(epilogue) if epilogue is not None else None
    _check(lib().fgemm_select_model(ctypes.byref(model), transA, transB, M, N, K, dtype, e,
                                    ctypes.byref(p)), "fgemm_select_model")
    return p


def fgemm_gemm(handle, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype,
               epilogue=None, stream=0, check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm(handle, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm")
    return s


def fgemm_gemm_plan(handle, plan, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                    dtype, epilogue=None, stream=0, check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm_plan(handle, ctypes.byref(plan), transA, transB, M, N, K, alpha, A, lda,
                              B, ldb, beta, C, ldc, dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm_plan")
    return s


def fgemm_gemm_noalloc(handle, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                       dtype, epilogue=None, stream=0, check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm_noalloc(handle, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                 ldc, dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm_noalloc")
    return s


def fgemm_gemm_f8(handle, M, N, K, alpha, A, lda, a_format, scale_a, B, ldb, b_format, scale_b,
                  beta, C, ldc, dtype, epilogue=None, stream=0, check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm_f8(handle, M, N, K, alpha, A, lda, a_format, scale_a, B, ldb, b_format,
                            scale_b, beta, C, ldc, dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm_f8")
    return s


def fgemm_gemm_mxf8(handle, M, N, K, alpha, A, lda, a_format, a_scales, ld_a_scales, B, ldb,
                    b_format, b_scales, ld_b_scales, beta, C, ldc, dtype, epilogue=None,
                    stream=0, check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm_mxf8(handle, M, N, K, alpha, A, lda, a_format, a_scales, ld_a_scales, B,
                              ldb, b_format, b_scales, ld_b_scales, beta, C, ldc, dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm_mxf8")
    return s


def fgemm_gemm_mxf4(handle, M, N, K, alpha, A, lda, a_scales, ld_a_scales, B, ldb, b_scales,
                    ld_b_scales, beta, C, ldc, dtype, epilogue=None, stream=0,
                    check=True) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    s = lib().fgemm_gemm_mxf4(handle, M, N, K, alpha, A, lda, a_scales, ld_a_scales, B, ldb,
                              b_scales, ld_b_scales, beta, C, ldc, dtype, e, stream)
    if check:
        _check(s, "fgemm_gemm_mxf4")
    return s


def fgemm_quantize_mx(X, rows, cols, ldx, x_dtype, transpose, fmt, Q, ldq, scales, ld_scales,
                      stream=0, check=True) -> int:
    s = lib().fgemm_quantize_mx(X, rows, cols, ldx, x_dtype, int(bool(transpose)), fmt, Q, ldq,
                                scales, ld_scales, stream)
    if check:
        _check(s, "fgemm_quantize_mx")
    return s


def quantize_mx(X, fmt, *, transpose=False, Q=None, scales=None, stream=None):
    """MX quantization of a 2-D fp16/bf16 device tensor by fgemm_quantize_mx: blocks of
    32 along its rows, or (transpose) along its columns, i.e. of X^T.  Returns (Q,
    scales): uint8 codes of X or X^T (two E2M1 values a byte) and E8M0 scales whose
    row stride is rounded up to whole 16-byte groups, as the MX GEMMs take them."""
    import torch
    rows, cols = X.shape
    orows, olen = (cols, rows) if transpose else (rows, cols)
    width = olen // 2 if fmt == FGEMM_E2M1 else olen
    if Q is None:
        Q = torch.empty((orows, width), dtype=torch.uint8, device=X.device)
    if scales is None:
        scols = max(16, (olen // 32 + 15) // 16 * 16)
        scales = torch.full((orows, scols), 127, dtype=torch.uint8, device=X.device)
    s = current_stream() if stream is None else stream
    fgemm_quantize_mx(X.data_ptr(), rows, cols, _ld(X), torch_dtype_code(X), transpose, fmt,
                      Q.data_ptr(), _ld(Q), scales.data_ptr(), _ld(scales), s)
    return Q, scales


def fgemm_check_args(transA, transB, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype,
                     epilogue=None) -> int:
    e = ctypes.byref(epilogue) if epilogue is not None else None
    return lib().fgemm_check_args(transA, transB, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype, e)


def fgemm_tile_count(M, N, tile_m, tile_n) -> int:
    return lib().fgemm_tile_count(M, N, tile_m, tile_n)


def fgemm_wave_count(tiles, units):
    tail = ctypes.c_double()
    w = lib().fgemm_wave_count(tiles, units, ctypes.byref(tail))
    return w, tail.value


def fgemm_plan_rel_err(dtype, plan) -> float:
    return lib().fgemm_plan_rel_err(dtype, ctypes.byref(plan))


def fgemm_read_probe(src, nbytes, out, stream=None, check=True) -> int:
    s = lib().fgemm_read_probe(src, nbytes, out, stream)
    if check:
        _check(s, "fgemm_read_probe")
    return s


# ------------------------------------------------------------ torch conveniences
def torch_dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FGEMM_BF16
    if t.dtype == torch.float16:
        return FGEMM_F16
    raise TypeError(f"fgemm takes fp16 or bf16 tensors, not {t.dtype}")


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ld(t) -> int:
    if t.dim() != 2:
        raise ValueError("operands are 2-D row-major tensors (unit column stride)")
    if t.numel() == 0:  # an empty operand (K = 0): any leading dimension >= its width
        return max(t.shape[1], 1)
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("operands are 2-D row-major tensors (unit column stride)")
    return t.stride(0)


class Handle:
    """Owns an fgemm handle on one device."""

    def __init__(self, device: int = 0):
        self.h = fgemm_create(device)

    def close(self):
        if self.h:
            fgemm_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def gemm(self, A, B, C, *, transA=False, transB=False, alpha=1.0, beta=0.0, epilogue=None,
             plan=None, stream=None, noalloc=False):
        """C = alpha*op(A)*op(B) + beta*C on torch device tensors (C written in place);
        noalloc: through fgemm_gemm_noalloc (fixed device scratch, no allocation)."""
        ta = FGEMM_OP_T if transA else FGEMM_OP_N
        tb = FGEMM_OP_T if transB else FGEMM_OP_N
        M = A.shape[1] if transA else A.shape[0]
        K = A.shape[0] if transA else A.shape[1]
        N = C.shape[1]
        if epilogue is not None and epilogue.flags & FGEMM_EPI_SWIGLU_BWD:
            N //= 2  # the backward writes the gate and up gradients: C is M x 2N
        dt = torch_dtype_code(C)
        s = current_stream() if stream is None else stream
        args = (ta, tb, M, N, K, float(alpha), A.data_ptr(), _ld(A), B.data_ptr(), _ld(B),
                float(beta), C.data_ptr(), _ld(C), dt, epilogue, s)
        if noalloc:
            if plan is not None:
                raise ValueError("fgemm_gemm_noalloc takes no plan")
            return fgemm_gemm_noalloc(self.h, *args)
        if plan is None:
            return fgemm_gemm(self.h, *args)
        return fgemm_gemm_plan(self.h, plan, *args)

    def gemm_f8(self, A, B, C, *, a_format=FGEMM_E4M3, b_format=FGEMM_E4M3, scale_a=1.0,
                scale_b=1.0, alpha=1.0, beta=0.0, epilogue=None, stream=None):
        """C = alpha * (scale_a*A) (scale_b*B)^T + beta*C on torch device tensors: A
        (M x K) and B (N x K) hold 8-bit codes (uint8 or a float8 dtype), C is 16-bit."""
        M, K = A.shape
        N = B.shape[0]
        s = current_stream() if stream is None else stream
        return fgemm_gemm_f8(self.h, M, N, K, float(alpha), A.data_ptr(), _ld(A), a_format,
                             float(scale_a), B.data_ptr(), _ld(B), b_format, float(scale_b),
                             float(beta), C.data_ptr(), _ld(C), torch_dtype_code(C), epilogue, s)

    def gemm_mxf8(self, A, B, C, a_scales, b_scales, *, a_format=FGEMM_E4M3,
                  b_format=FGEMM_E4M3, alpha=1.0, beta=0.0, epilogue=None, stream=None):
        """MXFP8: as gemm_f8 with E8M0 block scales, a_scales (M x >= K/32) and b_scales
        (N x >= K/32) uint8 device tensors."""
        M, K = A.shape
        N = B.shape[0]
        s = current_stream() if stream is None else stream
        return fgemm_gemm_mxf8(self.h, M, N, K, float(alpha), A.data_ptr(), _ld(A), a_format,
                               a_scales.data_ptr(), _ld(a_scales), B.data_ptr(), _ld(B), b_format,
                               b_scales.data_ptr(), _ld(b_scales), float(beta), C.data_ptr(),
                               _ld(C), torch_dtype_code(C), epilogue, s)

    def gemm_mxf4(self, A, B, C, a_scales, b_scales, *, alpha=1.0, beta=0.0, epilogue=None,
                  stream=None):
        """MXFP4: A (M x K/2) and B (N x K/2) uint8 device tensors of packed E2M1 values
        (two a byte), a_scales (M x >= K/32) and b_scales (N x >= K/32) E8M0 bytes;
        C = alpha * A' B'^T + beta * C."""
        M, K = A.shape[0], 2 * A.shape[1]
        N = B.shape[0]
        s = current_stream() if stream is None else stream
        return fgemm_gemm_mxf4(self.h, M, N, K, float(alpha), A.data_ptr(), _ld(A),
                               a_scales.data_ptr(), _ld(a_scales), B.data_ptr(), _ld(B),
                               b_scales.data_ptr(), _ld(b_scales), float(beta), C.data_ptr(),
                               _ld(C), torch_dtype_code(C), epilogue, s)

    def select(self, M, N, K, *, transA=False, transB=False, dtype=FGEMM_BF16, epilogue=None):
        return fgemm_select(self.h, FGEMM_OP_T if transA else FGEMM_OP_N,
                            FGEMM_OP_T if transB else FGEMM_OP_N, M, N, K, dtype, epilogue)

    def model(self) -> fgemm_model_t:
        return fgemm_get_model(self.h)


def read_probe(t, out=None, stream=None):
    """One streaming read of the device tensor `t` (contiguous, a multiple of 16 bytes,
    16-byte aligned) by fgemm_read_probe; returns the int32 tensor of the
    FGEMM_READ_PROBE_GROUPS per-workgroup XOR checksums."""
    import torch
    if not t.is_contiguous():
        raise ValueError("read_probe takes a contiguous tensor")
    if out is None:
        out = torch.empty(FGEMM_READ_PROBE_GROUPS, dtype=torch.int32, device=t.device)
    s = current_stream() if stream is None else stream
    fgemm_read_probe(t.data_ptr(), t.numel() * t.element_size(), out.data_ptr(), s)
    return out


def strassen_plan(depth: int, variant: int, tile: int = 0) -> fgemm_plan_t:
    p = fgemm_plan_t()
    p.path, p.depth, p.variant = FGEMM_PATH_STRASSEN, depth, variant
    p.tile_m = p.tile_n = tile
    return p


def classical_plan(tile_m: int = 0, tile_n: int = 0, split_k: int = 1) -> fgemm_plan_t:
    p = fgemm_plan_t()
    p.path, p.tile_m, p.tile_n, p.split_k = FGEMM_PATH_CLASSICAL, tile_m, tile_n, split_k
    return p
