"""GPU parity of the classical MFMA path against the CPU oracle, through the C ABI.

Exact cases use small-integer inputs whose products and sums are exact in fp32
and in the 16-bit output, so the GPU must match the oracle bit for bit.  Random
cases are held to the normwise bound ||C - Q(D)||_F / ||Q(D)||_F <= 1e-3."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import (BF16, CLASSICAL_TOL, F16, check_full, from_dev, handle, rel_err, run, say,
                      to_dev)

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]
TILES = [(256, 256), (128, 128), (64, 128), (32, 128), (64, 64)]


def stored(M, N, K, transA, transB, A_lo, seedA, seedB, dtype, kind="int"):
    shapeA = (K, M) if transA else (M, K)
    shapeB = (N, K) if transB else (K, N)
    if kind == "int":
        lo = -1 if dtype == BF16 else -2
        return (inputs.integers(shapeA, seedA, dtype, lo, -lo),
                inputs.integers(shapeB, seedB, dtype, lo, -lo))
    return inputs.normal(shapeA, seedA, dtype), inputs.normal(shapeB, seedB, dtype)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transA,transB", LAYOUTS)
def test_exact_integer_products(tile, dtype, transA, transB):
    # |C| <= K*max|a|*max|b| = 256 (bf16) / 1024 (fp16): exact in the output type
    # whole-phase K with ragged M/N (clamped fast path), K tails (checked path), tiny
    for (M, N, K) in [(256, 256, 256), (300, 200, 256), (33, 136, 128), (300, 200, 130),
                      (1, 264, 64), (67, 9, 1)]:
        say(f"exact tile={tile} dtype={dtype} tA={transA} tB={transB} M={M} N={N} K={K}")
        A, B = stored(M, N, K, transA, transB, 0, 11 + M, 12 + N, dtype)
        _, Q, _ = oracle.gemm(A, B, transA=transA, transB=transB, dtype=dtype)
        got = run(A, B, dtype, transA=transA, transB=transB, M=M, N=N,
                  plan=fgemm.classical_plan(*tile))
        assert np.array_equal(got, Q), (M, N, K)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("dtype", [BF16, F16])
def test_edge_chunk_straddling_the_matrix_edge(tile, dtype):
    """Aligned leading dimensions, but an M/N-contiguous operand whose edge dimension
    is not a multiple of 8: a 16-byte chunk of the edge tile straddles the edge and
    must not be moved (NN: B stored K x N with N = 77 and ldb = ldc = 80; TN: A
    stored K x M with M = 70 and lda = 72).  Integer inputs and an integer C with
    beta = 1: every output is exact, so the comparison is bitwise."""
    for (transA, M, N, K, pad) in [(False, 64, 77, 64, (0, 3, 3)), (True, 70, 64, 64, (2, 0, 0)),
                                   (False, 300, 205, 128, (0, 3, 3)),
                                   (True, 270, 136, 128, (2, 0, 0)),
                                   (True, 70, 77, 64, (2, 3, 3))]:
        say(f"edge chunk tile={tile} dtype={dtype} tA={transA} M={M} N={N} K={K} pad={pad}")
        A, B = stored(M, N, K, transA, False, 0, 15 + M, 16 + N, dtype)
        C = inputs.integers((M, N), 17 + K, dtype, -4, 4)
        _, Q, _ = oracle.gemm(A, B, transA=transA, beta=1.0, C=C, dtype=dtype)
        got = run(A, B, dtype, transA=transA, M=M, N=N, beta=1.0, C_bits=C, pad=pad,
                  plan=fgemm.classical_plan(*tile))
        assert np.array_equal(got, Q), (transA, M, N, K)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transA,transB", LAYOUTS)
def test_random_ragged_with_alpha_beta(dtype, transA, transB):
    M, N, K = 600, 520, 328   # several 256 tiles, ragged in every dimension
    say(f"random dtype={dtype} tA={transA} tB={transB}")
    A, B = stored(M, N, K, transA, transB, 0, 21, 22, dtype, kind="normal")
    C = inputs.normal((M, N), 23, dtype)
    _, Q, _ = oracle.gemm(A, B, transA=transA, transB=transB, alpha=0.75, beta=0.5, C=C,
                          dtype=dtype)
    for tile in TILES:
        got = run(A, B, dtype, transA=transA, transB=transB, alpha=0.75, beta=0.5, C_bits=C,
                  plan=fgemm.classical_plan(*tile))
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, tile
    got = run(A, B, dtype, transA=transA, transB=transB, alpha=0.75, beta=0.5, C_bits=C)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


@pytest.mark.parametrize("transA,transB", LAYOUTS)
def test_unaligned_leading_dimensions(transA, transB):
    # leading dimensions not a multiple of 8 take the element-wise path
    dtype = BF16
    M, N, K = 133, 77, 91
    say(f"unaligned tA={transA} tB={transB}")
    A, B = stored(M, N, K, transA, transB, 0, 31, 32, dtype, kind="normal")
    C = inputs.normal((M, N), 33, dtype)
    _, Q, _ = oracle.gemm(A, B, transA=transA, transB=transB, beta=-1.0, C=C, dtype=dtype)
    got = run(A, B, dtype, transA=transA, transB=transB, beta=-1.0, C_bits=C, pad=3)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


def test_k_zero_gives_beta_c():
    dtype = BF16
    M, N = 70, 90
    say("K=0")
    C = inputs.normal((M, N), 41, dtype)
    import torch
    Cd = to_dev(C, dtype)
    A = torch.empty((M, 1), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    st = fgemm.fgemm_gemm(handle().h, 0, 0, M, N, 0, 1.0, A.data_ptr(), 1, B.data_ptr(), N, 0.5,
                          Cd.data_ptr(), N, fgemm.FGEMM_BF16, None, fgemm.current_stream())
    assert st == 0
    torch.cuda.synchronize()
    ref = oracle.encode(0.5 * oracle.decode(C, dtype), dtype)
    assert np.array_equal(from_dev(Cd), ref)


def test_beta_zero_never_reads_c_and_alpha_zero():
    dtype = F16
    M, N, K = 96, 80, 64
    say("beta=0 with NaN C; alpha=0")
    A, B = stored(M, N, K, False, False, 0, 51, 52, dtype, kind="normal")
    got = run(A, B, dtype, C_bits=np.full((M, N), 0x7E00, dtype=np.uint16))
    assert np.isfinite(oracle.decode(got, dtype)).all()
    C = inputs.normal((M, N), 53, dtype)
    got = run(A, B, dtype, alpha=0.0, beta=2.0, C_bits=C)
    assert np.array_equal(got, oracle.encode(2.0 * oracle.decode(C, dtype), dtype))


def test_identity_and_transpose_invariants():
    dtype = BF16
    say("A*I = A and (AB)^T = B^T A^T")
    A = inputs.normal((200, 136), 61, dtype)
    I = inputs.to_bits(np.eye(136), dtype)
    assert np.array_equal(run(A, I, dtype), A)
    B = inputs.integers((136, 72), 62, dtype, -1, 1)
    Ai = inputs.integers((200, 136), 63, dtype, -1, 1)
    AB = run(Ai, B, dtype)
    BtAt = run(B, Ai, dtype, transA=True, transB=True, M=72, N=200)
    assert np.array_equal(BtAt, AB.T)


def test_repeatable_bitwise():
    dtype = BF16
    say("repeatability 1024^3")
    A = inputs.normal((1024, 1024), 71, dtype)
    B = inputs.normal((1024, 1024), 72, dtype)
    r1 = run(A, B, dtype)
    r2 = run(A, B, dtype)
    assert np.array_equal(r1, r2)


# ------------------------------------------------------------ workload sizes
def test_fp16_256_cube():
    """fp16 NN row-major 256^3, U[-1,1] seeds 1001/1002, alpha=1 beta=0."""
    dtype = F16
    say("fp16 256^3")
    A = inputs.uniform((256, 256), 1001, dtype)
    B = inputs.uniform((256, 256), 1002, dtype)
    _, Q, _ = oracle.gemm(A, B, dtype=dtype)
    got = run(A, B, dtype)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


@pytest.mark.parametrize("n", [4096, 8192])
@pytest.mark.parametrize("transA", [False, True])
def test_bf16_square_beta_half(n, transA):
    """bf16 M=N=K in {4096, 8192}, NN and TN, N(0,1), alpha=1, beta=0.5, C N(0,1):
    full-size run with the library's own plan, every element of the output against
    the oracle's fp64 product within its rounding-error bound, and normwise."""
    dtype = BF16
    say(f"bf16 square n={n} transA={transA}")
    A = inputs.normal((n, n), 2001, dtype)
    B = inputs.normal((n, n), 2002, dtype)
    C = inputs.normal((n, n), 2003, dtype)
    got = run(A, B, dtype, transA=transA, beta=0.5, C_bits=C)
    D, S = oracle.gemm_dense(A, B, transA=transA, beta=0.5, C=C, dtype=dtype)
    check_full(got, D, S, n, dtype)


@pytest.mark.parametrize("M,N", [(16384, 4096), (16384, 14336), (1, 14336), (16, 14336),
                                 (64, 14336)])
def test_llm_shapes(M, N):
    """bf16 NN, activations N(0,1), weights N(0,0.02), K=4096; whole output."""
    dtype = BF16
    K = 4096
    say(f"llm M={M} N={N}")
    X = inputs.normal((M, K), 3001, dtype)
    W = inputs.normal((K, N), 3002, dtype, std=0.02)
    got = run(X, W, dtype)
    D, S = oracle.gemm_dense(X, W, dtype=dtype)
    check_full(got, D, S, K, dtype)


@pytest.mark.parametrize("tile", [(64, 64), (32, 128), (64, 128), (128, 128), (256, 256)])
@pytest.mark.parametrize("split", [2, 4])
@pytest.mark.parametrize("dtype", [BF16, F16])
def test_split_k_exact_and_random(tile, split, dtype):
    # exact: integer inputs, K = 256; random: beta and bias through the finalize pass
    for (M, N) in [(1, 264), (16, 520), (100, 136)]:
        K = 256
        say(f"split-K tile={tile} split={split} dtype={dtype} M={M} N={N}")
        A, B = stored(M, N, K, False, False, 0, 81 + M, 82 + N, dtype)
        _, Q, _ = oracle.gemm(A, B, dtype=dtype)
        got = run(A, B, dtype, M=M, N=N, plan=fgemm.classical_plan(*tile, split_k=split))
        assert np.array_equal(got, Q), (M, N)
    M, N, K = 48, 392, 512
    A, B = stored(M, N, K, False, True, 0, 91, 92, dtype, kind="normal")
    C = inputs.normal((M, N), 93, dtype)
    _, Q, _ = oracle.gemm(A, B, transB=True, alpha=0.5, beta=-0.75, C=C, dtype=dtype)
    got = run(A, B, dtype, transB=True, alpha=0.5, beta=-0.75, C_bits=C,
              plan=fgemm.classical_plan(*tile, split_k=split))
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


@pytest.mark.parametrize("tile", [(64, 64), (32, 128), (256, 256)])
@pytest.mark.parametrize("transB", [False, True])
@pytest.mark.parametrize("dtype", [BF16, F16])
def test_split_k_transposed_a_with_bias_and_beta(tile, transB, dtype):
    """Split K with A stored K x M: alpha, beta*C and bias applied once, in the
    finalize pass, after the fp32 slices are summed."""
    M, N, K = 40, 264, 512
    say(f"split-K transA tile={tile} tB={transB} dtype={dtype}")
    A, B = stored(M, N, K, True, transB, 0, 95, 96, dtype, kind="normal")
    C = inputs.normal((M, N), 97, dtype)
    bias = inputs.normal((N,), 98, dtype)
    _, Q, _ = oracle.gemm(A, B, transA=True, transB=transB, alpha=1.5, beta=0.25, C=C,
                          dtype=dtype, epi=oracle.EPI_BIAS, bias=bias)
    bd = to_dev(bias[None, :], dtype)
    for split in (2, 4):
        got = run(A, B, dtype, transA=True, transB=transB, alpha=1.5, beta=0.25, C_bits=C,
                  plan=fgemm.classical_plan(*tile, split_k=split),
                  epilogue=fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr()))
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, split


def test_split_k_refusals():
    import torch
    dtype = BF16
    say("split-K refusals")
    A = to_dev(inputs.normal((16, 96), 1, dtype), dtype)
    B = to_dev(inputs.normal((96, 64), 2, dtype), dtype)
    C = to_dev(np.zeros((16, 64), dtype=np.uint16), dtype)
    ssd = torch.zeros(16, dtype=torch.float32, device="cuda")
    # 96 = 3 phases of 32: not divisible into 2 slices
    st = fgemm.fgemm_gemm_plan(handle().h, fgemm.classical_plan(128, 128, split_k=2), 0, 0, 16,
                               64, 96, 1.0, A.data_ptr(), 96, B.data_ptr(), 64, 0.0, C.data_ptr(),
                               64, fgemm.FGEMM_BF16, None, fgemm.current_stream(), check=False)
    assert st == fgemm.FGEMM_ERR_NOT_SUPPORTED
    # the row-statistics epilogue needs the unsplit kernel
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=ssd.data_ptr())
    st = fgemm.fgemm_gemm_plan(handle().h, fgemm.classical_plan(32, 128, split_k=2), 0, 0, 16, 64,
                               96, 1.0, A.data_ptr(), 96, B.data_ptr(), 64, 0.0, C.data_ptr(), 64,
                               fgemm.FGEMM_BF16, epi, fgemm.current_stream(), check=False)
    assert st == fgemm.FGEMM_ERR_NOT_SUPPORTED
    torch.cuda.synchronize()


@pytest.mark.parametrize("tile,bk", [((256, 256), 64), ((128, 128), 32), ((64, 128), 32),
                                     ((32, 128), 64), ((64, 64), 64)])
@pytest.mark.parametrize("phases", [3, 5])
def test_persistent_chains_odd_and_even_phases(tile, bk, phases):
    """More tiles than the device holds at once, so every workgroup runs several tiles
    back to back (each tile's first loads issued by its predecessor); odd and even
    phase counts.  Integer inputs: exact."""
    dtype = BF16
    M = N = 4352
    K = phases * bk
    say(f"persistent chains tile={tile} K={K}")
    A, B = stored(M, N, K, False, False, 0, 101 + phases, 102 + phases, dtype)
    _, Q, _ = oracle.gemm(A, B, dtype=dtype)
    got = run(A, B, dtype, plan=fgemm.classical_plan(*tile))
    assert np.array_equal(got, Q)
    if tile == (256, 256):
        At, Bt = stored(M, N, K, True, True, 0, 103 + phases, 104 + phases, dtype)
        _, Qt, _ = oracle.gemm(At, Bt, transA=True, transB=True, dtype=dtype)
        got = run(At, Bt, dtype, transA=True, transB=True, M=M, N=N,
                  plan=fgemm.classical_plan(*tile))
        assert np.array_equal(got, Qt)


@pytest.mark.parametrize("transA", [False, True])
@pytest.mark.parametrize("edge8", [True, False])
def test_persistent_chains_through_edge_tiles(transA, edge8):
    """Chains of tiles per workgroup that cross edge tiles in one launch, with every
    leading dimension a multiple of 8 (the aligned kernel).  edge8: the M/N-contiguous
    operand's edge dimension is a multiple of 8, so its edge tiles stay on the
    direct-load path with clamped chunks; otherwise they take the bounds-checked
    path between direct-load tiles.  Integer inputs: exact."""
    dtype = BF16
    ragged = 4360 if edge8 else 4356  # 17 tiles of 256 plus 8 (or 4) rows or columns
    M, N, K = (4452, ragged, 320) if not transA else (ragged, 4452, 320)
    say(f"persistent chains with edge tiles transA={transA} M={M} N={N} K={K}")
    A, B = stored(M, N, K, transA, False, 0, 111, 112, dtype)
    _, Q, _ = oracle.gemm(A, B, transA=transA, dtype=dtype)
    # pad every operand to a leading dimension that is a multiple of 8
    pa = (-(M if transA else K)) % 8
    pb = (-N) % 8
    got = run(A, B, dtype, transA=transA, M=M, N=N, pad=(pa, pb, pb),
              plan=fgemm.classical_plan(256, 256))
    assert np.array_equal(got, Q)
