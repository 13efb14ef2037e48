"""GPU parity of the table-driven block scheme <2,2,3;11> (FGEMM_VARIANT_R223: op(A) in
2 x 2 blocks, op(B) and C in 2 x 3, eleven products) against the CPU oracle.  Integer
inputs must give the oracle's result bit for bit (scaled fp16 sums of small integers,
fp32 products and the rounding are exact there); random inputs are held to the
Strassen bounds, normwise and per element, and to the scheme's error-model figure."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import (BF16, F16, STRASSEN_TOL, check_full_strassen, from_dev, handle, rel_err,
                      run, say, to_dev)

pytestmark = pytest.mark.gpu

R223 = fgemm.FGEMM_VARIANT_R223
LAYOUTS = [(False, False), (True, False), (False, True), (True, True)]


def operands(M, N, K, transA, transB, seed, dtype, kind):
    shapeA = (K, M) if transA else (M, K)
    shapeB = (N, K) if transB else (K, N)
    if kind == "int":
        lo = -1 if dtype == BF16 else -2
        return (inputs.integers(shapeA, seed, dtype, lo, -lo),
                inputs.integers(shapeB, seed + 1, dtype, lo, -lo))
    return inputs.uniform(shapeA, seed, dtype), inputs.uniform(shapeB, seed + 1, dtype)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transA,transB", LAYOUTS)
def test_exact_integers(dtype, transA, transB):
    """Every layout, both tiles of the products, two shapes (one block of 16 x 16 x 16
    elements per product, and several tiles a product)."""
    for (M, N, K) in [(32, 48, 32), (256, 384, 320)]:
        say(f"r223 exact dtype={dtype} tA={transA} tB={transB} {M}x{N}x{K}")
        A, B = operands(M, N, K, transA, transB, 300 + M + K, dtype, "int")
        _, Q, _ = oracle.gemm(A, B, transA=transA, transB=transB, dtype=dtype)
        for tile in (256, 128):
            got = run(A, B, dtype, transA=transA, transB=transB, M=M, N=N,
                      plan=fgemm.strassen_plan(1, R223, tile))
            assert np.array_equal(got, Q), (M, N, K, tile)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transA,transB", LAYOUTS)
def test_random_with_beta_bias_and_padding(dtype, transA, transB):
    """U[-1,1] operands with alpha, beta*C and bias, every leading dimension 8 wider
    than its rows: within the Strassen bound and the scheme's error-model figure."""
    import torch
    M, N, K = 512, 768, 640
    say(f"r223 random dtype={dtype} tA={transA} tB={transB}")
    A, B = operands(M, N, K, transA, transB, 310, dtype, "uniform")
    C = inputs.normal((M, N), 312, dtype)
    bias = inputs.normal((N,), 313, dtype)
    _, Q, _ = oracle.gemm(A, B, transA=transA, transB=transB, alpha=0.75, beta=-0.5, C=C,
                          dtype=dtype, epi=oracle.EPI_BIAS, bias=bias)
    Ad, Bd, Cd = to_dev(A, dtype, 8), to_dev(B, dtype, 8), to_dev(C, dtype, 8)
    bd = to_dev(bias[None, :], dtype)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr())
    plan = fgemm.strassen_plan(1, R223)
    handle().gemm(Ad, Bd, Cd, transA=transA, transB=transB, alpha=0.75, beta=-0.5, epilogue=epi,
                  plan=plan)
    torch.cuda.synchronize()
    err = rel_err(from_dev(Cd), Q, dtype)
    assert err <= STRASSEN_TOL
    assert err <= fgemm.fgemm_plan_rel_err(dtype, plan)


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_large_whole_output(dtype):
    """8192 x 12288 x 8192, U[-1,1]: every element against the oracle's fp64 product."""
    M, N, K = 8192, 12288, 8192
    say(f"r223 large {M}x{N}x{K} dtype={dtype}")
    A = inputs.uniform((M, K), 5101, dtype)
    B = inputs.uniform((K, N), 5102, dtype)
    got = run(A, B, dtype, plan=fgemm.strassen_plan(1, R223))
    D, _ = oracle.gemm_dense(A, B, dtype=dtype, bound=False)
    worst = check_full_strassen(got, D, dtype)
    say(f"  largest element error {worst:.3g} x RMS(D)")


def test_refusals_and_plan_error():
    """Shapes that do not split into 16-element blocks, epilogues other than NONE and
    BIAS, and depth 2 are refused before anything is enqueued; the error model's
    figure exists for depth 1 only."""
    import torch
    say("r223 refusals")
    h = handle()
    A = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda")
    ss = torch.zeros(64, dtype=torch.float32, device="cuda")
    p1, p2 = fgemm.strassen_plan(1, R223), fgemm.strassen_plan(2, R223)
    s = fgemm.current_stream()

    def call(plan, Bt, Ct, epi=None):
        return fgemm.fgemm_gemm_plan(h.h, plan, 0, 0, 64, Ct.shape[1], 64, 1.0, A.data_ptr(), 64,
                                     Bt.data_ptr(), Bt.shape[1], 0.0, Ct.data_ptr(), Ct.shape[1],
                                     fgemm.FGEMM_BF16, epi, s, check=False)
    assert call(p1, B, C) == fgemm.FGEMM_OK
    B2 = torch.zeros((64, 80), dtype=torch.bfloat16, device="cuda")
    C2 = torch.zeros((64, 80), dtype=torch.bfloat16, device="cuda")
    assert call(p1, B2, C2) == fgemm.FGEMM_ERR_NOT_SUPPORTED       # N = 80: not 3 x 16k
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=ss.data_ptr())
    assert call(p1, B, C, epi) == fgemm.FGEMM_ERR_NOT_SUPPORTED    # statistics
    assert call(p2, B, C) == fgemm.FGEMM_ERR_INVALID_VALUE         # depth 2
    torch.cuda.synchronize()
    assert fgemm.fgemm_plan_rel_err(fgemm.FGEMM_BF16, p1) > 0
    assert fgemm.fgemm_plan_rel_err(fgemm.FGEMM_BF16, p2) < 0


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("dist", ["uniform", "normal"])
def test_error_model_calibration(dtype, dist):
    """The scheme's figure in the accuracy guard (fgemm_plan_rel_err) against
    measurement on i.i.d. 1024 x 1536 x 1024 inputs: the normwise error against
    RNE(D) is at most the figure and at least half of it."""
    M, N, K = 1024, 1536, 1024
    say(f"r223 error model dtype={dtype} dist={dist}")
    gen = inputs.uniform if dist == "uniform" else inputs.normal
    A, B = gen((M, K), 671, dtype), gen((K, N), 672, dtype)
    rows = inputs.sample_rows(M, 96, 13)
    _, Q, _ = oracle.gemm(A, B, dtype=dtype, rows=rows)
    plan = fgemm.strassen_plan(1, R223)
    pred = fgemm.fgemm_plan_rel_err(dtype, plan)
    err = rel_err(run(A, B, dtype, plan=plan)[rows], Q, dtype)
    say(f"  measured {err:.3e}, figure {pred:.3e}")
    assert 0.5 * pred <= err <= pred, (err, pred)
