"""GPU parity of the 8-bit GEMM (fgemm_gemm_f8: FP8 E4M3/E5M2 with per-tensor
scales, CS336 Lecture 05 notes, Page 27) against the CPU oracle, through the C ABI.

Small integers are exact in both 8-bit formats and their products and sums are
exact in fp32 and in the 16-bit output, so those cases must match the oracle bit for
bit.  Scaled random inputs are held to ||C - Q(D)||_F / ||Q(D)||_F <= 1e-3, and row
statistics to 1e-3."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import (BF16, CLASSICAL_TOL, F16, STATS_TOL, check_full, from_dev, handle, rel_err, say,
                      to_dev)

pytestmark = pytest.mark.gpu

E4, E5 = fgemm.FGEMM_E4M3, fgemm.FGEMM_E5M2
FORMATS = [(E4, E4), (E4, E5), (E5, E4), (E5, E5)]


def dev8(codes, pad=0):
    """uint8 codes -> device tensor, rows widened by `pad` bytes (filled with NaN codes)."""
    import torch
    codes = np.ascontiguousarray(codes)
    if pad:
        wide = np.full((codes.shape[0], codes.shape[1] + pad), 0x7F, dtype=np.uint8)
        wide[:, :codes.shape[1]] = codes
        return torch.from_numpy(wide).cuda()[:, :codes.shape[1]]
    return torch.from_numpy(codes.copy()).cuda()


def run8(A, B, dtype, *, fa=E4, fb=E4, sa=1.0, sb=1.0, alpha=1.0, beta=0.0, C_bits=None,
         epilogue=None, pad=(0, 0, 0)):
    import torch
    M, N = A.shape[0], B.shape[0]
    Ad, Bd = dev8(A, pad[0]), dev8(B, pad[1])
    if C_bits is None:
        C_bits = np.full((M, N), 0x7FC0 if dtype == BF16 else 0x7E00, dtype=np.uint16)
    Cd = to_dev(C_bits, dtype, pad[2])
    handle().gemm_f8(Ad, Bd, Cd, a_format=fa, b_format=fb, scale_a=sa, scale_b=sb, alpha=alpha,
                     beta=beta, epilogue=epilogue)
    torch.cuda.synchronize()
    return from_dev(Cd)


@pytest.mark.parametrize("fa,fb", FORMATS)
@pytest.mark.parametrize("dtype", [BF16, F16])
def test_exact_integers_every_phase_count(fa, fb, dtype):
    """Integer inputs: bitwise equal to the oracle, for 1 to 7 phases of 128 k (the
    three-stage ring's prologue, odd and even phase counts, and the copy that ends
    an odd run), ragged M and N, power-of-two scales and alpha, beta*C with an
    integer C."""
    lo = -1 if dtype == BF16 else -2
    for (M, N, K) in [(256, 128, 128), (300, 200, 256), (1, 264, 384), (64, 77, 512),
                      (130, 136, 640), (257, 129, 768), (33, 40, 896)]:
        say(f"f8 exact fa={fa} fb={fb} dtype={dtype} {M}x{N}x{K}")
        kk = min(K, 256)  # keep |C| within the 16-bit types' exact integers
        A = inputs.f8_integers((M, K), 3 + M, fa, lo, -lo)
        B = inputs.f8_integers((N, K), 4 + N, fb, lo, -lo)
        if K > kk:  # zero all but the first 256 columns of k
            A[:, kk:] = 0
        C = inputs.integers((M, N), 5 + K, dtype, -3, 3)
        _, Q, _ = oracle.gemm_f8(A, B, fmt_a=fa, fmt_b=fb, scale_a=0.5, scale_b=4.0, alpha=0.5,
                                 beta=1.0, C=C, dtype=dtype)
        pad_c = (-N) % 8
        got = run8(A, B, dtype, fa=fa, fb=fb, sa=0.5, sb=4.0, alpha=0.5, beta=1.0, C_bits=C,
                   pad=(0, 0, pad_c))
        assert np.array_equal(got, Q), (M, N, K)


@pytest.mark.parametrize("fa,fb", FORMATS)
@pytest.mark.parametrize("dtype", [BF16, F16])
def test_random_scaled_with_bias_and_row_statistics(fa, fb, dtype):
    """Per-tensor scaled N(0,1) activations and N(0,0.02) weights (the amax scale of
    Page 27), alpha, beta*C, bias and the row sums of squares; rows of A and B
    padded by 16 bytes."""
    import torch
    M, N, K = 600, 520, 384
    say(f"f8 random fa={fa} fb={fb} dtype={dtype}")
    A, sa = inputs.f8_normal((M, K), 61, fa)
    B, sb = inputs.f8_normal((N, K), 62, fb, std=0.02)
    C = inputs.normal((M, N), 63, dtype)
    bias = inputs.normal((N,), 64, dtype, std=0.1)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ
    _, Q, ss = oracle.gemm_f8(A, B, fmt_a=fa, fmt_b=fb, scale_a=sa, scale_b=sb, alpha=1.5,
                              beta=0.5, C=C, dtype=dtype, epi=flags, bias=bias)
    bd = to_dev(bias[None, :], dtype)
    ssd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ, bias=bd.data_ptr(),
                              rowsumsq=ssd.data_ptr())
    got = run8(A, B, dtype, fa=fa, fb=fb, sa=sa, sb=sb, alpha=1.5, beta=0.5, C_bits=C,
               epilogue=epi, pad=(16, 16, 0))
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL
    ssg = ssd.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ssg - ss) / ss) <= STATS_TOL


def test_persistent_chains_exact():
    """More tiles than the device holds at once (17 x 34 tiles of 256 x 128), so
    every workgroup runs several tiles back to back with the next tile's first
    phases loaded during the epilogue; odd and even phase counts.  Exact."""
    dtype = BF16
    M = N = 4352
    for K in (640, 768):
        say(f"f8 chains K={K}")
        A = inputs.f8_integers((M, K), 71, E4, -1, 1)
        B = inputs.f8_integers((N, K), 72, E4, -1, 1)
        A[:, 256:] = 0
        _, Q, _ = oracle.gemm_f8(A, B, dtype=dtype)
        got = run8(A, B, dtype)
        assert np.array_equal(got, Q), K


def test_llm_projection_shape_whole_output():
    """16384 tokens x 4096 -> 4096 (the projection shape), E4M3 activations and
    weights with per-tensor scales: every element against the oracle's fp64
    product within its rounding-error bound, and normwise."""
    dtype = BF16
    M, N, K = 16384, 4096, 4096
    say("f8 16384x4096x4096")
    A, sa = inputs.f8_normal((M, K), 3001, E4)
    B, sb = inputs.f8_normal((N, K), 3002, E4, std=0.02)
    got = run8(A, B, dtype, sa=sa, sb=sb)
    D, S = oracle.gemm_f8_dense(A, B, scale_a=sa, scale_b=sb)
    check_full(got, D, S, K, dtype)


def test_mx_llm_projection_shape_whole_output():
    """The projection shape in MXFP8 (E8M0 scale per 32 values): whole output."""
    dtype = BF16
    M, N, K = 16384, 4096, 4096
    say("mx 16384x4096x4096")
    A, sA = inputs.mx_normal((M, K), 3003, E4)
    B, sB = inputs.mx_normal((N, K), 3004, E4, std=0.02)
    got = run_mx(A, sA, B, sB, dtype)
    D, S = oracle.gemm_f8_dense(A, B, mx_a=sA, mx_b=sB)
    check_full(got, D, S, K, dtype)


def test_refusals():
    import torch
    say("f8 refusals")
    h = handle()
    A = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    B = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    s = fgemm.current_stream()

    def call(M=64, N=64, K=256, lda=256, ldb=256, ldc=64, fa=E4, fb=E4, dt=fgemm.FGEMM_BF16,
             epi=None, sa=1.0):
        return fgemm.fgemm_gemm_f8(h.h, M, N, K, 1.0, A.data_ptr(), lda, fa, sa, B.data_ptr(), ldb,
                                   fb, 1.0, 0.0, C.data_ptr(), ldc, dt, epi, s, check=False)
    assert call() == fgemm.FGEMM_OK
    assert call(K=192) == fgemm.FGEMM_ERR_NOT_SUPPORTED        # not whole 128-deep phases
    assert call(lda=264) == fgemm.FGEMM_ERR_NOT_SUPPORTED      # rows not 16-byte aligned
    assert call(lda=128) == fgemm.FGEMM_ERR_INVALID_VALUE      # lda < K
    assert call(fa=2) == fgemm.FGEMM_ERR_INVALID_VALUE
    assert call(sa=float("inf")) == fgemm.FGEMM_ERR_INVALID_VALUE
    assert call(sa=1e-39) == fgemm.FGEMM_ERR_NOT_SUPPORTED     # alpha*sa*sb below fp32 normals
    ssd = torch.ones(64, dtype=torch.float32, device="cuda")
    sw = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=ssd.data_ptr(), rms_n=64)
    assert call(epi=sw) == fgemm.FGEMM_ERR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert bool((C == 0).all())


# ------------------------------------------------------------------ MXFP8 block scales
def run_mx(A, sA, B, sB, dtype, *, fa=E4, fb=E4, alpha=1.0, beta=0.0, C_bits=None, epilogue=None):
    import torch
    M, N = A.shape[0], B.shape[0]
    Ad, Bd, sAd, sBd = dev8(A), dev8(B), dev8(sA), dev8(sB)
    if C_bits is None:
        C_bits = np.full((M, N), 0x7FC0 if dtype == BF16 else 0x7E00, dtype=np.uint16)
    pad_c = (-N) % 8
    Cd = to_dev(C_bits, dtype, pad_c)
    handle().gemm_mxf8(Ad, Bd, Cd, sAd, sBd, a_format=fa, b_format=fb, alpha=alpha, beta=beta,
                       epilogue=epilogue)
    torch.cuda.synchronize()
    return from_dev(Cd)


@pytest.mark.parametrize("fa,fb", FORMATS)
def test_mx_exact_integers_every_group(fa, fb):
    """Integer codes with random E8M0 block scales in 2^-3..2^3: every product and
    partial sum is exact in fp32, so the GPU result must equal the oracle's
    rounding of the exact sum bit for bit.  1 to 9 phases of 128 k cover the first
    scale group, the switch between the two group buffers and a partial last group."""
    dtype = BF16
    for (M, N, K) in [(256, 128, 128), (300, 200, 512), (64, 77, 640), (257, 129, 1024),
                      (33, 40, 1152)]:
        say(f"mx exact fa={fa} fb={fb} {M}x{N}x{K}")
        A, sA = inputs.mx_integers((M, K), 81 + M, fa, -2, 2)
        B, sB = inputs.mx_integers((N, K), 82 + N, fb, -2, 2)
        C = inputs.integers((M, N), 83 + K, dtype, -3, 3)
        _, Q, _ = oracle.gemm_f8(A, B, fmt_a=fa, fmt_b=fb, mx_a=sA, mx_b=sB, alpha=0.5, beta=1.0,
                                 C=C, dtype=dtype)
        got = run_mx(A, sA, B, sB, dtype, fa=fa, fb=fb, alpha=0.5, beta=1.0, C_bits=C)
        assert np.array_equal(got, Q), (M, N, K)


def test_mx_persistent_chains_exact():
    """MX with more tiles than the device holds at once (17 x 34 tiles of 256 x 128):
    the next tile's first scale group is loaded while other waves finish the last
    phase, whose group sits in either buffer (4, 5 and 9 phases).  Exact."""
    dtype = BF16
    M = N = 4352
    for K in (512, 640, 1152):
        say(f"mx chains K={K}")
        A, sA = inputs.mx_integers((M, K), 171, E4, -1, 1)
        B, sB = inputs.mx_integers((N, K), 172, E4, -1, 1)
        A[:, 256:] = 0
        _, Q, _ = oracle.gemm_f8(A, B, mx_a=sA, mx_b=sB, dtype=dtype)
        got = run_mx(A, sA, B, sB, dtype)
        assert np.array_equal(got, Q), K


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_mx_random_block_scaled_with_statistics(dtype):
    """Block-scaled N(0,1) activations and N(0,0.02) weights (every 32 values their
    own power-of-two scale), bias and row sums of squares; within 1e-3."""
    import torch
    M, N, K = 600, 520, 1024
    say(f"mx random dtype={dtype}")
    A, sA = inputs.mx_normal((M, K), 91, E4)
    B, sB = inputs.mx_normal((N, K), 92, E4, std=0.02)
    bias = inputs.normal((N,), 94, dtype, std=0.1)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ
    _, Q, ss = oracle.gemm_f8(A, B, mx_a=sA, mx_b=sB, dtype=dtype, epi=flags, bias=bias)
    bd = to_dev(bias[None, :], dtype)
    ssd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ, bias=bd.data_ptr(),
                              rowsumsq=ssd.data_ptr())
    got = run_mx(A, sA, B, sB, dtype, epilogue=epi)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL
    ssg = ssd.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ssg - ss) / ss) <= STATS_TOL


def test_mx_refusals():
    import torch
    say("mx refusals")
    h = handle()
    A = torch.zeros((64, 512), dtype=torch.uint8, device="cuda")
    S = torch.full((64, 32), 127, dtype=torch.uint8, device="cuda")
    C = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    s = fgemm.current_stream()

    def call(K=512, lds=16, sp=S.data_ptr()):
        return fgemm.fgemm_gemm_mxf8(h.h, 64, 64, K, 1.0, A.data_ptr(), 512, E4, sp, lds,
                                     A.data_ptr(), 512, E4, sp, lds, 0.0, C.data_ptr(), 64,
                                     fgemm.FGEMM_BF16, None, s, check=False)
    assert call() == fgemm.FGEMM_OK
    assert call(lds=8) == fgemm.FGEMM_ERR_INVALID_VALUE        # fewer than K/32 scales a row
    assert call(lds=24) == fgemm.FGEMM_ERR_NOT_SUPPORTED       # not whole 16-byte groups
    assert call(K=384, lds=12) == fgemm.FGEMM_ERR_NOT_SUPPORTED
    assert call(sp=0) == fgemm.FGEMM_ERR_INVALID_VALUE
    torch.cuda.synchronize()
