"""GPU parity of the MXFP4 GEMM (fgemm_gemm_mxf4: E2M1 values with E8M0 scales per
32 values, CS336 Lecture 05 notes, Page 29) against the CPU oracle, through the C ABI.

Values of magnitude <= 2 with block scales 2^-2..2^2 are multiples of 2^-6 whose
sums over K <= 2304 stay inside fp32's 24 bits, so the GPU's fp32 sums are
exact and those cases must match the oracle's rounding bit for bit.  Block-scaled
normal inputs are held to ||C - Q(D)||_F / ||Q(D)||_F <= 1e-3, every output of the
LLM shape to its elementwise fp32 bound, and row statistics to 1e-3."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import (BF16, CLASSICAL_TOL, F16, STATS_TOL, check_full, from_dev, handle, rel_err,
                      say, to_dev)

pytestmark = pytest.mark.gpu


def dev_bytes(a, pad=0, fill=0x77):
    """uint8 rows -> device tensor, rows widened by `pad` bytes of `fill` (0x77 is two
    6.0 values: a read past a row's end shows in the product)."""
    import torch
    a = np.ascontiguousarray(a)
    if pad:
        wide = np.full((a.shape[0], a.shape[1] + pad), fill, dtype=np.uint8)
        wide[:, :a.shape[1]] = a
        return torch.from_numpy(wide).cuda()[:, :a.shape[1]]
    return torch.from_numpy(a.copy()).cuda()


def run_f4(A, sA, B, sB, dtype, *, alpha=1.0, beta=0.0, C_bits=None, epilogue=None, pad=0):
    import torch
    M, N = A.shape[0], B.shape[0]
    Ad, Bd = dev_bytes(A, pad), dev_bytes(B, pad)
    sAd, sBd = dev_bytes(sA), dev_bytes(sB)
    if C_bits is None:
        C_bits = np.full((M, N), 0x7FC0 if dtype == BF16 else 0x7E00, dtype=np.uint16)
    Cd = to_dev(C_bits, dtype, (-N) % 8)
    handle().gemm_mxf4(Ad, Bd, Cd, sAd, sBd, alpha=alpha, beta=beta, epilogue=epilogue)
    torch.cuda.synchronize()
    return from_dev(Cd)


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_exact_every_phase_count(dtype):
    """1 to 9 phases of 256 values (the two-stage ring's prologue, the first scale
    group of two phases, the switch between the two group buffers, a partial last
    group), ragged M and N, rows padded with 6.0 values, alpha and beta*C with an
    integer C: bitwise."""
    for (M, N, K, pad) in [(256, 128, 256, 0), (300, 200, 1024, 16), (64, 77, 1280, 0),
                           (257, 129, 2048, 32), (33, 40, 2304, 0), (1, 264, 768, 16)]:
        say(f"mxf4 exact dtype={dtype} {M}x{N}x{K} pad={pad}")
        A, sA = inputs.mxf4_small((M, K), 11 + M)
        B, sB = inputs.mxf4_small((N, K), 12 + N)
        C = inputs.integers((M, N), 13 + K, dtype, -3, 3)
        _, Q, _ = oracle.gemm_mxf4(A, B, sA, sB, alpha=0.5, beta=1.0, C=C, dtype=dtype)
        got = run_f4(A, sA, B, sB, dtype, alpha=0.5, beta=1.0, C_bits=C, pad=pad)
        assert np.array_equal(got, Q), (M, N, K)


def test_every_code_and_extreme_scales():
    """A's first block holds all 16 codes twice, B random codes, block scales from
    2^-20 to 2^20; A's other blocks are zero, so every output is one block's exact
    product sum times its two scales."""
    dtype = BF16
    M, N, K = 64, 64, 256
    say("mxf4 every code")
    rng = np.random.default_rng(5)
    ca = np.tile(np.arange(16, dtype=np.uint8), (M, K // 16))
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sA = np.full((M, 16), 127, np.uint8)
    sB = np.full((N, 16), 127, np.uint8)
    sA[:, :K // 32] = rng.integers(107, 148, size=(M, K // 32))
    sB[:, :K // 32] = rng.integers(107, 148, size=(N, K // 32))
    ca[:, 32:] = 0           # one block of A per row: one product sum per output
    A, B = inputs.pack_f4_codes(ca), inputs.pack_f4_codes(cb)
    _, Q, _ = oracle.gemm_mxf4(A, B, sA, sB, dtype=dtype)
    got = run_f4(A, sA, B, sB, dtype)
    assert np.array_equal(got, Q)


def test_persistent_chains_exact():
    """More 256 x 256 tiles than the device holds at once (17 x 17): the next tile's
    first phases and scale group load while the current tile finishes, with 2, 3 and
    5 phases a tile.  Exact."""
    dtype = BF16
    M = N = 4352
    for K in (512, 768, 1280):
        say(f"mxf4 chains K={K}")
        A, sA = inputs.mxf4_small((M, K), 171)
        B, sB = inputs.mxf4_small((N, K), 172)
        _, Q, _ = oracle.gemm_mxf4(A, B, sA, sB, dtype=dtype)
        got = run_f4(A, sA, B, sB, dtype)
        assert np.array_equal(got, Q), K


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_random_block_scaled_with_bias_and_statistics(dtype):
    """MXFP4-quantized N(0,1) activations and N(0,0.02) weights, bias and the row
    sums of squares: within 1e-3 normwise and 1e-3 for the statistics."""
    import torch
    M, N, K = 600, 520, 1024
    say(f"mxf4 random dtype={dtype}")
    A, sA = inputs.mxf4_normal((M, K), 91)
    B, sB = inputs.mxf4_normal((N, K), 92, std=0.02)
    bias = inputs.normal((N,), 94, dtype, std=0.1)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ
    _, Q, ss = oracle.gemm_mxf4(A, B, sA, sB, dtype=dtype, epi=flags, bias=bias)
    bd = to_dev(bias[None, :], dtype)
    ssd = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ, bias=bd.data_ptr(),
                              rowsumsq=ssd.data_ptr())
    got = run_f4(A, sA, B, sB, dtype, epilogue=epi)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL
    ssg = ssd.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ssg - ss) / ss) <= STATS_TOL


def test_llm_projection_shape_whole_output():
    """16384 tokens x 4096 -> 4096 in MXFP4: every element against the oracle's
    fp64 product within its rounding-error bound, and normwise."""
    dtype = BF16
    M, N, K = 16384, 4096, 4096
    say("mxf4 16384x4096x4096")
    A, sA = inputs.mxf4_normal((M, K), 3005)
    B, sB = inputs.mxf4_normal((N, K), 3006, std=0.02)
    got = run_f4(A, sA, B, sB, dtype)
    D, S = oracle.gemm_mxf4_dense(A, B, sA, sB)
    check_full(got, D, S, K, dtype)


def test_k_zero_and_refusals():
    import torch
    say("mxf4 refusals")
    h = handle()
    A = torch.zeros((64, 256), dtype=torch.uint8, device="cuda")   # K = 512 values a row
    S = torch.full((64, 16), 127, dtype=torch.uint8, device="cuda")
    C = torch.full((64, 64), 2.0, dtype=torch.bfloat16, device="cuda")
    s = fgemm.current_stream()

    def call(K=512, lda=256, lds=16, sp=S.data_ptr(), beta=0.0, dt=fgemm.FGEMM_BF16):
        return fgemm.fgemm_gemm_mxf4(h.h, 64, 64, K, 1.0, A.data_ptr(), lda, sp, lds,
                                     A.data_ptr(), lda, sp, lds, beta, C.data_ptr(), 64, dt, None,
                                     s, check=False)
    assert call(K=0, sp=0, lds=0, beta=0.5) == fgemm.FGEMM_OK     # C = 0.5 * C, no scale read
    torch.cuda.synchronize()
    assert bool((C == 1.0).all())
    assert call() == fgemm.FGEMM_OK
    torch.cuda.synchronize()
    assert bool((C == 0).all())
    assert call(K=384, lds=16) == fgemm.FGEMM_ERR_NOT_SUPPORTED    # not whole 256-value phases
    assert call(lda=264) == fgemm.FGEMM_ERR_NOT_SUPPORTED          # rows not 16-byte aligned
    assert call(lda=128) == fgemm.FGEMM_ERR_INVALID_VALUE          # fewer than K/2 bytes a row
    assert call(lds=8) == fgemm.FGEMM_ERR_INVALID_VALUE            # fewer than K/32 scales a row
    assert call(lds=24) == fgemm.FGEMM_ERR_NOT_SUPPORTED           # not whole 16-byte groups
    assert call(sp=0) == fgemm.FGEMM_ERR_INVALID_VALUE
    assert call(dt=7) == fgemm.FGEMM_ERR_INVALID_VALUE
    torch.cuda.synchronize()
