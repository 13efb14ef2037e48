"""GPU parity of the MX quantizer (fgemm_quantize_mx: CS336 Lecture 05 notes, Page 27:
q = cast(x/s) with an E8M0 scale per 32 values; Pages 27-28: the transpose quantized
on its own) against the CPU oracle, through the C ABI.  Codes and scales are bytes,
so every case must match the oracle bit for bit."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import BF16, CLASSICAL_TOL, F16, from_dev, handle, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [fgemm.FGEMM_E4M3, fgemm.FGEMM_E5M2, fgemm.FGEMM_E2M1]


def gpu_quantize(X_bits, dtype, fmt, transpose, pad=0):
    """Quantize on the device; returns (Q, S) cut to the oracle's shapes (the
    library's scale rows are padded to whole 16-byte groups)."""
    import torch
    X = to_dev(X_bits, dtype, pad)
    Q, S = fgemm.quantize_mx(X, fmt, transpose=transpose)
    torch.cuda.synchronize()
    rows, cols = X_bits.shape
    olen = rows if transpose else cols
    return Q.cpu().numpy(), S.cpu().numpy()[:, :olen // 32]


def special_matrix(rows, cols, dtype, seed):
    """N(0,1) values with some rows scaled by 2^-30..2^14 (fp16: 2^-12..2^10), one
    all-zero block, negative values that round to -0, and exact format values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols))
    lo, hi = (-30, 14) if dtype == BF16 else (-12, 10)
    x *= np.exp2(rng.integers(lo, hi, size=(rows, 1)))
    x[0, :32] = 0.0
    if rows > 1 and cols >= 64:
        x[1, 32:64] = 1.0
        x[1, 32] = -1e-6          # -> -0 next to the block's 1.0 values
        x[1, 33] = 448.0 if dtype == BF16 else 6.0
    return inputs.to_bits(x, dtype)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transpose", [False, True])
def test_bitwise_ragged_shapes(fmt, dtype, transpose):
    """Shapes that leave partial tiles (and, transposed, a column count that is not a
    multiple of 8), padded source rows, and the special blocks: codes and scales
    equal the oracle's."""
    shapes = [(96, 77), (288, 200), (32, 8)] if transpose else [(77, 96), (300, 224), (1, 32)]
    for (rows, cols) in shapes:
        for pad in ((-cols) % 8, (-cols) % 8 + 8):   # row strides that stay multiples of 8
            say(f"quantize fmt={fmt} dtype={dtype} T={transpose} {rows}x{cols} pad={pad}")
            X = special_matrix(rows, cols, dtype, 7 + rows + cols)
            Qo, So = oracle.quantize_mx(X, dtype, fmt, transpose=transpose)
            Qg, Sg = gpu_quantize(X, dtype, fmt, transpose, pad)
            assert np.array_equal(Sg, So), (rows, cols)
            assert np.array_equal(Qg, Qo), (rows, cols)


@pytest.mark.parametrize("fmt,transpose,shape", [
    (fgemm.FGEMM_E4M3, False, (16384, 4096)),     # activations of the projection shape
    (fgemm.FGEMM_E2M1, True, (4096, 14336))])     # FFN-up weights W (K x N) -> W^T (N x K)
def test_full_size_llm_operands(fmt, transpose, shape):
    dtype = BF16
    say(f"quantize full size fmt={fmt} T={transpose} {shape}")
    std = 0.02 if transpose else 1.0
    X = inputs.normal(shape, 3001 + fmt, dtype, std=std)
    Qo, So = oracle.quantize_mx(X, dtype, fmt, transpose=transpose)
    Qg, Sg = gpu_quantize(X, dtype, fmt, transpose)
    assert np.array_equal(Sg, So)
    assert np.array_equal(Qg, Qo)


@pytest.mark.parametrize("fmt", [fgemm.FGEMM_E4M3, fgemm.FGEMM_E2M1])
def test_quantize_then_gemm(fmt):
    """Activations X (M x K) quantized row-wise and weights W (K x N, row-major)
    quantized transposed on the device, then the MX GEMM: within 1e-3 of the
    oracle's product of the oracle's quantization of the same matrices."""
    import torch
    dtype = BF16
    M, N, K = 512, 384, 1024
    say(f"quantize then gemm fmt={fmt}")
    X = inputs.normal((M, K), 61, dtype)
    W = inputs.normal((K, N), 62, dtype, std=0.02)
    Xd, Wd = to_dev(X, dtype), to_dev(W, dtype)
    qa, sa = fgemm.quantize_mx(Xd, fmt)
    qb, sb = fgemm.quantize_mx(Wd, fmt, transpose=True)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if fmt == fgemm.FGEMM_E2M1:
        handle().gemm_mxf4(qa, qb, C, sa, sb)
    else:
        handle().gemm_mxf8(qa, qb, C, sa, sb, a_format=fmt, b_format=fmt)
    torch.cuda.synchronize()
    QA, SA = oracle.quantize_mx(X, dtype, fmt)
    QB, SB = oracle.quantize_mx(W, dtype, fmt, transpose=True)
    if fmt == fgemm.FGEMM_E2M1:
        _, Q, _ = oracle.gemm_mxf4(QA, QB, SA, SB, dtype=dtype)
    else:
        _, Q, _ = oracle.gemm_f8(QA, QB, fmt_a=fmt, fmt_b=fmt, mx_a=SA, mx_b=SB, dtype=dtype)
    assert rel_err(from_dev(C), Q, dtype) <= CLASSICAL_TOL


def test_refusals_and_empty():
    import torch
    say("quantize refusals")
    X = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    Q = torch.zeros((64, 64), dtype=torch.uint8, device="cuda")
    S = torch.zeros((64, 16), dtype=torch.uint8, device="cuda")
    s = fgemm.current_stream()

    def call(rows=64, cols=64, ldx=64, dt=fgemm.FGEMM_BF16, tr=0, fmt=fgemm.FGEMM_E4M3, q=None,
             ldq=64, lds=16, x=None):
        return fgemm.fgemm_quantize_mx(x if x is not None else X.data_ptr(), rows, cols, ldx, dt,
                                       tr, fmt, q if q is not None else Q.data_ptr(), ldq,
                                       S.data_ptr(), lds, s, check=False)
    assert call() == fgemm.FGEMM_OK
    assert call(cols=48, ldx=64) == fgemm.FGEMM_ERR_INVALID_VALUE   # row length % 32
    assert call(tr=1, rows=48) == fgemm.FGEMM_ERR_INVALID_VALUE     # transposed: rows % 32
    assert call(ldq=32) == fgemm.FGEMM_ERR_INVALID_VALUE            # shorter than a row
    assert call(lds=1) == fgemm.FGEMM_ERR_INVALID_VALUE             # fewer scales than blocks
    assert call(fmt=3) == fgemm.FGEMM_ERR_INVALID_VALUE
    assert call(dt=7) == fgemm.FGEMM_ERR_INVALID_VALUE
    assert call(ldx=60, cols=32) == fgemm.FGEMM_ERR_NOT_SUPPORTED   # rows not 16-byte aligned
    assert call(ldq=72) == fgemm.FGEMM_ERR_NOT_SUPPORTED            # ldq % 16
    assert call(rows=0) == fgemm.FGEMM_OK                            # nothing to do
    torch.cuda.synchronize()
