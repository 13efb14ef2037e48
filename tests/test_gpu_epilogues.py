"""GPU parity of the fused epilogues (bias, per-row sum of squares, RMS row scale +
SwiGLU) and of the two-GEMM chain that uses them, against the CPU oracle."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import (BF16, CLASSICAL_TOL, F16, STATS_TOL, check_full, from_dev, handle, rel_err, say,
                      to_dev, empty_out)

pytestmark = pytest.mark.gpu
TILES = [(256, 256), (128, 128), (64, 128), (32, 128), (64, 64)]


def dev_f32(n, fill=np.nan):
    import torch
    return torch.full((n,), fill, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("tile", TILES)
def test_bias_and_rowsumsq(dtype, tile):
    import torch
    M, N, K = 300, 520, 200
    say(f"bias+rowsumsq dtype={dtype} tile={tile}")
    A = inputs.normal((M, K), 81, dtype)
    B = inputs.normal((K, N), 82, dtype, std=0.1)
    C = inputs.normal((M, N), 83, dtype)
    bias = inputs.normal((N,), 84, dtype)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ
    _, Q, ss = oracle.gemm(A, B, beta=0.25, C=C, dtype=dtype, epi=flags, bias=bias)
    Ad, Bd, Cd, bd = to_dev(A, dtype), to_dev(B, dtype), to_dev(C, dtype), to_dev(bias[None, :], dtype)
    ssd = dev_f32(M)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ, bias=bd.data_ptr(),
                              rowsumsq=ssd.data_ptr())
    handle().gemm(Ad, Bd, Cd, beta=0.25, epilogue=epi, plan=fgemm.classical_plan(*tile))
    torch.cuda.synchronize()
    assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL
    got = ssd.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ss) / ss) <= STATS_TOL


def test_rowsumsq_exact_constant_rows():
    # K = 1 and a row of ones: every output row is constant, ss = N * a_i^2 exactly
    import torch
    dtype = BF16
    M, N = 130, 4096
    say("rowsumsq constant rows")
    a = inputs.integers((M, 1), 85, dtype, -3, 3)
    ones = inputs.to_bits(np.ones((1, N)), dtype)
    ssd = dev_f32(M)
    Cd = empty_out(M, N, dtype)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=ssd.data_ptr())
    handle().gemm(to_dev(a, dtype), to_dev(ones, dtype), Cd, epilogue=epi)
    torch.cuda.synchronize()
    av = oracle.decode(a, dtype)[:, 0]
    assert np.array_equal(ssd.cpu().numpy().astype(np.float64), N * av * av)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transB", [False, True])
@pytest.mark.parametrize("tile", TILES[:3])
def test_rms_swiglu_ragged(dtype, transB, tile):
    import torch
    M, K, Nout = 300, 256, 264
    say(f"rms_swiglu dtype={dtype} transB={transB} tile={tile}")
    X = inputs.normal((M, K), 91, dtype)
    W = inputs.normal((K, 2 * Nout), 92, dtype, std=0.1)
    ss = (np.random.default_rng(93).uniform(0.5, 2.0, M) * 4096).astype(np.float32)
    C = inputs.normal((M, Nout), 94, dtype)
    _, Q, _ = oracle.gemm(X, W, dtype=dtype, epi=oracle.EPI_RMS_SWIGLU, rms_ss=ss.astype(np.float64),
                          rms_n=4096, rms_eps=1e-6, beta=0.5, C=C, alpha=1.5)
    Wst = np.ascontiguousarray(W.T) if transB else W
    Xd, Wd, Cd = to_dev(X, dtype), to_dev(Wst, dtype), to_dev(C, dtype)
    ssd = torch.from_numpy(ss).cuda()
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=ssd.data_ptr(), rms_n=4096,
                              rms_eps=1e-6)
    handle().gemm(Xd, Wd, Cd, transB=transB, alpha=1.5, beta=0.5, epilogue=epi,
                  plan=fgemm.classical_plan(*tile))
    torch.cuda.synchronize()
    assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL


def run_chain(M, H, F, seed0, dtype=BF16):
    """GEMM1 X[M x H] W[H x H] + row sums of squares; GEMM2 Y W2[H x 2F] + RMS + SwiGLU."""
    import torch
    X = inputs.normal((M, H), seed0, dtype)
    W = inputs.normal((H, H), seed0 + 1, dtype, std=0.02)
    W2 = inputs.normal((H, 2 * F), seed0 + 2, dtype, std=0.02)
    Xd, Wd, W2d = to_dev(X, dtype), to_dev(W, dtype), to_dev(W2, dtype)
    Yd = empty_out(M, H, dtype)
    ssd = dev_f32(M)
    Od = empty_out(M, F, dtype)
    e1 = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=ssd.data_ptr())
    e2 = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=ssd.data_ptr(), rms_n=H,
                             rms_eps=1e-6)
    handle().gemm(Xd, Wd, Yd, epilogue=e1)
    handle().gemm(Yd, W2d, Od, epilogue=e2)
    torch.cuda.synchronize()
    return X, W, W2, from_dev(Yd), ssd.cpu().numpy().astype(np.float64), from_dev(Od)


def check_chain(X, W, W2, Y, ss, O, rows, H, dtype=BF16):
    _, Yq, ssr = oracle.gemm(X, W, dtype=dtype, epi=oracle.EPI_ROWSUMSQ, rows=rows)
    assert rel_err(Y[rows], Yq, dtype) <= CLASSICAL_TOL
    assert np.max(np.abs(ss[rows] - ssr) / ssr) <= STATS_TOL
    # GEMM2 on the oracle's own Y rows and statistics
    _, Oq, _ = oracle.gemm(Yq, W2, dtype=dtype, epi=oracle.EPI_RMS_SWIGLU, rms_ss=ssr, rms_n=H,
                           rms_eps=1e-6)
    assert rel_err(O[rows], Oq, dtype) <= CLASSICAL_TOL


def test_chain_small_full_check():
    say("chain 520x384 -> 2x264")
    X, W, W2, Y, ss, O = run_chain(520, 384, 264, 4100)
    check_chain(X, W, W2, Y, ss, O, np.arange(520), 384)


def test_chain_llm_size():
    """M=8192, hidden 4096, FFN 11008: X N(0,1), W and W2 N(0,0.02).  Sampled rows
    through the ascending-k oracle, then every element of Y and of the SwiGLU
    output against the fp64 references within their rounding-error bounds (GEMM2
    on the Y and statistics it was given), and every row's statistics."""
    dtype, M, H = BF16, 8192, 4096
    say("chain 8192x4096 -> 2x11008")
    X, W, W2, Y, ss, O = run_chain(M, H, 11008, 4001)
    check_chain(X, W, W2, Y, ss, O, inputs.sample_rows(M, 24, 9), H)
    D1, S1 = oracle.gemm_dense(X, W, dtype=dtype)
    check_full(Y, D1, S1, H, dtype)
    y = oracle.decode(Y, dtype)
    assert np.max(np.abs(ss - np.sum(y * y, axis=1)) / ss) <= STATS_TOL
    D2, E2 = oracle.rms_swiglu_dense(Y, W2, rms_ss=ss, rms_n=H, rms_eps=1e-6, dtype=dtype,
                                     bound=True)
    # fp32 sums (gamma E2 to first order), a few ulps of fp32 in the row scale, the
    # exponential and the products, then the 16-bit rounding
    n = H + 4
    gamma = n * 2.0 ** -23 / (1 - n * 2.0 ** -23)
    u16 = 2.0 ** -8
    bound = u16 * np.abs(D2) + (1 + u16) * (gamma * E2 + 8 * 2.0 ** -23 * np.abs(D2))
    o = oracle.decode(O, dtype)
    bad = ~(np.abs(o - D2) <= bound)
    assert not bad.any(), f"{int(bad.sum())} SwiGLU outputs outside the bound"
    assert rel_err(O, oracle.encode(D2, dtype), dtype) <= CLASSICAL_TOL


# ------------------------------------------------------------ activation and RoPE
ACTS = [fgemm.FGEMM_ACT_RELU, fgemm.FGEMM_ACT_SILU, fgemm.FGEMM_ACT_GELU_TANH]
ORACLE_ACT = {fgemm.FGEMM_ACT_RELU: oracle.ACT_RELU, fgemm.FGEMM_ACT_SILU: oracle.ACT_SILU,
              fgemm.FGEMM_ACT_GELU_TANH: oracle.ACT_GELU_TANH}


def run_transform(A, B, C, dtype, epi, plan=None, transB=False, alpha=1.0, beta=0.0, pad=0,
                  M=None):
    import torch
    Ad, Bd = to_dev(A, dtype, pad), to_dev(B, dtype, pad)
    Cd = to_dev(C, dtype, pad) if C is not None else empty_out(M, B.shape[0] if transB else B.shape[1], dtype)
    handle().gemm(Ad, Bd, Cd, transB=transB, alpha=alpha, beta=beta, epilogue=epi, plan=plan)
    torch.cuda.synchronize()
    return from_dev(Cd)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("tile", TILES)
def test_activation_bias_rowsumsq(dtype, act, tile):
    """D = act(alpha*acc + beta*C + bias) before the rounding, statistics of the
    written rows; ragged in every dimension."""
    import torch
    M, N, K = 300, 520, 200
    say(f"activation dtype={dtype} act={act} tile={tile}")
    A = inputs.normal((M, K), 701, dtype)
    B = inputs.normal((K, N), 702, dtype, std=0.1)
    C = inputs.normal((M, N), 703, dtype)
    bias = inputs.normal((N,), 704, dtype)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ | oracle.EPI_ACT
    _, Q, ss = oracle.gemm(A, B, alpha=1.25, beta=0.25, C=C, dtype=dtype, epi=flags, bias=bias,
                           act=ORACLE_ACT[act])
    Ad, Bd, Cd, bd = to_dev(A, dtype), to_dev(B, dtype), to_dev(C, dtype), to_dev(bias[None, :], dtype)
    ssd = dev_f32(M)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ | fgemm.FGEMM_EPI_ACT,
                              bias=bd.data_ptr(), rowsumsq=ssd.data_ptr(), act=act)
    handle().gemm(Ad, Bd, Cd, alpha=1.25, beta=0.25, epilogue=epi, plan=fgemm.classical_plan(*tile))
    torch.cuda.synchronize()
    assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL
    got = ssd.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ss) / ss) <= STATS_TOL


def test_relu_exact_integers():
    # integer products: ReLU of exact integers is exact, bit for bit on every tile
    dtype = BF16
    M, N, K = 130, 264, 64
    A = inputs.integers((M, K), 711, dtype, -1, 1)
    B = inputs.integers((K, N), 712, dtype, -1, 1)
    _, Q, _ = oracle.gemm(A, B, dtype=dtype, epi=oracle.EPI_ACT, act=oracle.ACT_RELU)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ACT, act=fgemm.FGEMM_ACT_RELU)
    for tile in TILES:
        say(f"relu exact tile={tile}")
        got = run_transform(A, B, None, dtype, epi, plan=fgemm.classical_plan(*tile), M=M)
        assert np.array_equal(got, Q), tile


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_bias_pointer_off_16_bytes_exact(dtype):
    """Aligned operands with a bias vector that starts 2 bytes past a 16-byte boundary
    (the epilogue loads it element by element), beta*C, alpha and the row sums of
    squares, on tiles whose interior waves take the whole-block store and whose edge
    waves take the general one: integer values, so the outputs are exact and must
    match the oracle bit for bit; the statistics within 1e-3."""
    import torch
    M, N, K = 300, 520, 192
    A = inputs.integers((M, K), 741, dtype, -2, 2)
    B = inputs.integers((K, N), 742, dtype, -2, 2)
    C = inputs.integers((M, N), 743, dtype, -4, 4)
    bias = inputs.integers((N + 1,), 744, dtype, -3, 3)
    flags = oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ
    _, Q, ss = oracle.gemm(A, B, alpha=0.5, beta=1.5, C=C, dtype=dtype, epi=flags, bias=bias[1:])
    bd = to_dev(bias[None, :], dtype)
    assert (bd.data_ptr() + 2) % 16 != 0
    for tile in TILES:
        say(f"bias off 16 bytes dtype={dtype} tile={tile}")
        Ad, Bd, Cd = to_dev(A, dtype), to_dev(B, dtype), to_dev(C, dtype)
        ssd = dev_f32(M)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ,
                                  bias=bd.data_ptr() + 2, rowsumsq=ssd.data_ptr())
        handle().gemm(Ad, Bd, Cd, alpha=0.5, beta=1.5, epilogue=epi,
                      plan=fgemm.classical_plan(*tile))
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(Cd), Q), tile
        got = ssd.cpu().numpy().astype(np.float64)
        nz = ss > 0
        assert np.max(np.abs(got[nz] - ss[nz]) / ss[nz]) <= STATS_TOL, tile
        assert np.all(got[~nz] == 0), tile


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("transB", [False, True])
def test_rope_positions_and_offset(dtype, tile, transB):
    """Interleaved-pair rotary embedding of alpha*acc + bias, head width 64, with a
    position array (values up to 8191) and with row index + offset."""
    import torch
    M, K, hd, heads = 300, 256, 64, 6
    N = hd * heads
    say(f"rope dtype={dtype} tile={tile} tB={transB}")
    X = inputs.normal((M, K), 721, dtype)
    W = inputs.normal((K, N), 722, dtype, std=0.05)
    bias = inputs.normal((N,), 723, dtype)
    pos = np.random.default_rng(724).integers(0, 8192, size=M).astype(np.int32)
    Wst = np.ascontiguousarray(W.T) if transB else W
    bd = to_dev(bias[None, :], dtype)
    posd = torch.from_numpy(pos).cuda()
    for mode in ("array", "offset"):
        if mode == "array":
            opos, epi = pos, fgemm.make_epilogue(
                fgemm.FGEMM_EPI_ROPE | fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr(),
                rope_positions=posd.data_ptr(), rope_head_dim=hd, rope_theta=10000.0)
        else:
            opos, epi = np.arange(M) + 5000, fgemm.make_epilogue(
                fgemm.FGEMM_EPI_ROPE | fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr(), rope_offset=5000,
                rope_head_dim=hd, rope_theta=10000.0)
        _, Q, _ = oracle.gemm(X, W, alpha=0.5, dtype=dtype, epi=oracle.EPI_ROPE | oracle.EPI_BIAS,
                              bias=bias, rope_pos=opos, rope_head_dim=hd, rope_theta=10000.0)
        got = run_transform(X, Wst, None, dtype, epi, plan=fgemm.classical_plan(*tile),
                            transB=transB, alpha=0.5, M=M)
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, mode


def test_transforms_unaligned_operands():
    # leading dimensions that are not multiples of 8: the register epilogue
    dtype = F16
    M, K, N = 70, 96, 128
    X = inputs.normal((M, K), 731, dtype)
    W = inputs.normal((K, N), 732, dtype, std=0.1)
    say("transforms unaligned")
    for epi_f, okw, gkw in (
            (oracle.EPI_ACT, dict(act=oracle.ACT_GELU_TANH),
             dict(act=fgemm.FGEMM_ACT_GELU_TANH)),
            (oracle.EPI_ROPE, dict(rope_pos=np.arange(M) + 77, rope_head_dim=32),
             dict(rope_offset=77, rope_head_dim=32))):
        _, Q, _ = oracle.gemm(X, W, dtype=dtype, epi=epi_f, **okw)
        flag = fgemm.FGEMM_EPI_ACT if epi_f == oracle.EPI_ACT else fgemm.FGEMM_EPI_ROPE
        got = run_transform(X, W, None, dtype, fgemm.make_epilogue(flag, **gkw), pad=3, M=M)
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, epi_f


def test_rope_llm_projection_size():
    """The projection shape 16384 tokens x 4096 -> 4096 with RoPE over 32 heads of
    128 (four sequences of 4096 positions), as the model picks the plan; sampled rows."""
    import torch
    dtype, M, K, N, hd = BF16, 16384, 4096, 4096, 128
    say("rope 16384x4096x4096")
    X = inputs.normal((M, K), 3001, dtype)
    W = inputs.normal((K, N), 3002, dtype, std=0.02)
    pos = (np.arange(M) % 4096).astype(np.int32)
    posd = torch.from_numpy(pos).cuda()
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROPE, rope_positions=posd.data_ptr(),
                              rope_head_dim=hd, rope_theta=10000.0)
    got = run_transform(X, W, None, dtype, epi, M=M)
    rows = inputs.sample_rows(M, 32, 11)
    _, Q, _ = oracle.gemm(X, W, dtype=dtype, epi=oracle.EPI_ROPE, rope_pos=pos, rope_head_dim=hd,
                          rows=rows)
    assert rel_err(got[rows], Q, dtype) <= CLASSICAL_TOL


def test_gelu_llm_ffn_up_size():
    """FFN up projection 16384 x 4096 -> 14336 with bias + GELU, as the model picks
    the plan; sampled rows."""
    import torch
    dtype, M, K, N = BF16, 16384, 4096, 14336
    say("gelu 16384x4096x14336")
    X = inputs.normal((M, K), 3001, dtype)
    W = inputs.normal((K, N), 3002, dtype, std=0.02)
    bias = inputs.normal((N,), 3003, dtype, std=0.02)
    bd = to_dev(bias[None, :], dtype)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ACT | fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr(),
                              act=fgemm.FGEMM_ACT_GELU_TANH)
    got = run_transform(X, W, None, dtype, epi, M=M)
    rows = inputs.sample_rows(M, 32, 12)
    _, Q, _ = oracle.gemm(X, W, dtype=dtype, epi=oracle.EPI_ACT | oracle.EPI_BIAS, bias=bias,
                          act=oracle.ACT_GELU_TANH, rows=rows)
    assert rel_err(got[rows], Q, dtype) <= CLASSICAL_TOL


def test_rope_backward_is_negated_positions():
    """The backward of RoPE is the rotation by the opposite angle: running the
    rotated output through an identity GEMM with negated positions gives back the
    unrotated product (to two roundings), and matches the oracle at -pos."""
    import torch
    dtype, M, K, hd, heads = F16, 256, 192, 64, 4
    N = hd * heads
    say("rope backward")
    X = inputs.normal((M, K), 741, dtype)
    W = inputs.normal((K, N), 742, dtype, std=0.1)
    pos = np.random.default_rng(743).integers(0, 4096, size=M).astype(np.int32)
    posd, negd = torch.from_numpy(pos).cuda(), torch.from_numpy(-pos).cuda()
    fwd = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROPE, rope_positions=posd.data_ptr(), rope_head_dim=hd)
    bwd = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROPE, rope_positions=negd.data_ptr(), rope_head_dim=hd)
    Y = run_transform(X, W, None, dtype, fwd, M=M)
    eye = inputs.to_bits(np.eye(N), dtype)
    back = run_transform(Y, eye, None, dtype, bwd, M=M)
    _, Q, _ = oracle.gemm(X, W, dtype=dtype)
    assert rel_err(back, Q, dtype) <= 2 * CLASSICAL_TOL
    _, Qb, _ = oracle.gemm(Y, eye, dtype=dtype, epi=oracle.EPI_ROPE, rope_pos=-pos.astype(np.int64),
                           rope_head_dim=hd)
    assert rel_err(back, Qb, dtype) <= CLASSICAL_TOL



# ------------------------------------------------------------ SwiGLU backward
def run_swiglu_bwd(X, W, dO, ss, dtype, transB=False, tile=None, alpha=1.0, pad=0):
    import torch
    M, Nout = dO.shape
    Xd, dOd = to_dev(X, dtype, pad), to_dev(dO, dtype, pad)
    Wst = np.ascontiguousarray(W.T) if transB else W
    Wd = to_dev(Wst, dtype, pad)
    Cd = empty_out(M, 2 * Nout, dtype)
    ssd = torch.from_numpy(np.asarray(ss, dtype=np.float32)).cuda()
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_SWIGLU_BWD, rms_rowsumsq=ssd.data_ptr(), rms_n=4096,
                              rms_eps=1e-6, swiglu_dout=dOd.data_ptr(), swiglu_ldd=dOd.stride(0))
    handle().gemm(Xd, Wd, Cd, transB=transB, alpha=alpha, epilogue=epi,
                  plan=fgemm.classical_plan(*tile) if tile else None)
    torch.cuda.synchronize()
    return from_dev(Cd)


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("transB", [False, True])
@pytest.mark.parametrize("tile", TILES[:3])
def test_swiglu_backward_ragged(dtype, transB, tile):
    """Gradient of the RMS + SwiGLU epilogue with respect to the recomputed gate|up
    product (row scale fixed), ragged M and N, against the oracle."""
    M, K, Nout = 300, 256, 264
    say(f"swiglu bwd dtype={dtype} transB={transB} tile={tile}")
    X = inputs.normal((M, K), 751, dtype)
    W = inputs.normal((K, 2 * Nout), 752, dtype, std=0.1)
    dO = inputs.normal((M, Nout), 753, dtype)
    ss = (np.random.default_rng(754).uniform(0.5, 2.0, M) * 4096).astype(np.float32)
    _, Q, _ = oracle.swiglu_bwd(X, W, dO, rms_ss=ss.astype(np.float64), rms_n=4096, rms_eps=1e-6,
                             alpha=1.5, dtype=dtype)
    got = run_swiglu_bwd(X, W, dO, ss, dtype, transB=transB, tile=tile, alpha=1.5)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


def test_swiglu_backward_unaligned():
    # leading dimensions that are not multiples of 8 take the bounds-checked loads
    dtype = BF16
    M, K, Nout = 70, 96, 64
    say("swiglu bwd unaligned")
    X = inputs.normal((M, K), 761, dtype)
    W = inputs.normal((K, 2 * Nout), 762, dtype, std=0.1)
    dO = inputs.normal((M, Nout), 763, dtype)
    ss = np.full(M, 4096.0, dtype=np.float32)
    _, Q, _ = oracle.swiglu_bwd(X, W, dO, rms_ss=ss.astype(np.float64), rms_n=4096, rms_eps=1e-6,
                             dtype=dtype)
    got = run_swiglu_bwd(X, W, dO, ss, dtype, pad=3)
    assert rel_err(got, Q, dtype) <= CLASSICAL_TOL


def test_swiglu_backward_llm_size():
    """The chain's second GEMM backward at its configured size: Y [8192 x 4096] N(0,1),
    W2 [4096 x 2*11008] N(0,0.02), dO N(0,1), as the model picks the plan; sampled rows."""
    dtype, M, K, Nout = BF16, 8192, 4096, 11008
    say("swiglu bwd 8192x4096 -> 2x11008")
    Y = inputs.normal((M, K), 4101, dtype)
    W2 = inputs.normal((K, 2 * Nout), 4102, dtype, std=0.02)
    dO = inputs.normal((M, Nout), 4103, dtype)
    ss = (np.random.default_rng(4104).uniform(0.5, 2.0, M) * K).astype(np.float32)
    got = run_swiglu_bwd(Y, W2, dO, ss, dtype)
    rows = inputs.sample_rows(M, 24, 14)
    _, Q, _ = oracle.swiglu_bwd(Y, W2, dO, rms_ss=ss[rows].astype(np.float64), rms_n=4096,
                             rms_eps=1e-6, dtype=dtype, rows=rows)
    assert rel_err(got[rows], Q, dtype) <= CLASSICAL_TOL



# ------------------------------------------------------------ RMSNorm backward
def run_rmsnorm_backward(Y, W2, dO, ss, dtype, tile=None):
    """SWIGLU_BWD with the row-scale gradient, then dY = dH W2^T + c_i Y (RMS_BWD)."""
    import torch
    M, H = Y.shape
    F = dO.shape[1]
    Yd, W2d, dOd = to_dev(Y, dtype), to_dev(W2, dtype), to_dev(dO, dtype)
    ssd = torch.from_numpy(np.asarray(ss, dtype=np.float32)).cuda()
    rg = dev_f32(M)
    dH = empty_out(M, 2 * F, dtype)
    e1 = fgemm.make_epilogue(fgemm.FGEMM_EPI_SWIGLU_BWD, rms_rowsumsq=ssd.data_ptr(), rms_n=H,
                             rms_eps=1e-6, swiglu_dout=dOd.data_ptr(), swiglu_ldd=F,
                             rms_grad=rg.data_ptr())
    plan = fgemm.classical_plan(*tile) if tile else None
    handle().gemm(Yd, W2d, dH, epilogue=e1, plan=plan)
    dY = empty_out(M, H, dtype)
    e2 = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_BWD, rms_rowsumsq=ssd.data_ptr(), rms_n=H,
                             rms_eps=1e-6, rms_grad=rg.data_ptr(), rms_x=Yd.data_ptr(), rms_ldx=H)
    handle().gemm(dH, W2d, dY, transB=True, epilogue=e2, plan=plan if tile != (64, 64) else None)
    torch.cuda.synchronize()
    return from_dev(dH), rg.cpu().numpy().astype(np.float64), from_dev(dY)


def check_rmsnorm_backward(Y, W2, dO, ss, dH, rg, dY, rows, dtype):
    H = Y.shape[1]
    _, Qh, rgr = oracle.swiglu_bwd(Y, W2, dO, rms_ss=ss[rows], rms_n=H, rms_eps=1e-6, dtype=dtype,
                                   rows=rows)
    assert rel_err(dH[rows], Qh, dtype) <= CLASSICAL_TOL
    assert np.linalg.norm(rg[rows] - rgr) <= STATS_TOL * np.linalg.norm(rgr)
    # dY against the oracle on the inputs it was given (the GPU's dH and scale gradient)
    _, Qy = oracle.rms_bwd(dH, W2, Y, rms_ss=ss[rows], rgrad=rg[rows], rms_n=H, rms_eps=1e-6,
                           transB=True, dtype=dtype, rows=rows)
    assert rel_err(dY[rows], Qy, dtype) <= CLASSICAL_TOL


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("tile", TILES[:3])
def test_rmsnorm_backward_ragged(dtype, tile):
    M, H, F = 300, 264, 136
    say(f"rmsnorm bwd dtype={dtype} tile={tile}")
    Y = inputs.normal((M, H), 771, dtype)
    W2 = inputs.normal((H, 2 * F), 772, dtype, std=0.1)
    dO = inputs.normal((M, F), 773, dtype)
    ss = np.sum(oracle.decode(Y, dtype) ** 2, axis=1)
    dH, rg, dY = run_rmsnorm_backward(Y, W2, dO, ss, dtype, tile=tile)
    check_rmsnorm_backward(Y, W2, dO, ss, dH, rg, dY, np.arange(M), dtype)


def test_rmsnorm_backward_llm_size():
    """The chain's backward at its configured size: Y [8192 x 4096], W2 [4096 x
    2*11008] N(0,0.02), dO N(0,1); both GEMMs as the model picks; sampled rows."""
    dtype, M, H, F = BF16, 8192, 4096, 11008
    say("rmsnorm bwd 8192x4096 / 2x11008")
    Y = inputs.normal((M, H), 4201, dtype)
    W2 = inputs.normal((H, 2 * F), 4202, dtype, std=0.02)
    dO = inputs.normal((M, F), 4203, dtype)
    ss = np.sum(oracle.decode(Y, dtype) ** 2, axis=1)
    dH, rg, dY = run_rmsnorm_backward(Y, W2, dO, ss, dtype)
    check_rmsnorm_backward(Y, W2, dO, ss, dH, rg, dY, inputs.sample_rows(M, 16, 15), dtype)


# ------------------------------------------------------------ degenerate shapes
def test_new_epilogues_degenerate_shapes():
    """K = 0 (the transforms act on beta*C + bias alone; the backward epilogues see
    a zero product), a single row, and tiny ragged shapes with K tails."""
    import torch
    dtype = BF16
    for (M, N, K) in [(5, 16, 0), (1, 24, 40), (3, 8, 3), (67, 40, 130)]:
        say(f"degenerate M={M} N={N} K={K}")
        A = inputs.normal((M, K), 781, dtype)
        B = inputs.normal((K, N), 782, dtype, std=0.2)
        C = inputs.normal((M, N), 783, dtype)
        bias = inputs.normal((N,), 784, dtype)
        bd = to_dev(bias[None, :], dtype)
        # activation with bias and beta
        _, Q, _ = oracle.gemm(A, B, beta=0.5, C=C, dtype=dtype, epi=oracle.EPI_ACT | oracle.EPI_BIAS,
                              bias=bias, act=oracle.ACT_GELU_TANH)
        got = run_transform(A, B, C, dtype, fgemm.make_epilogue(
            fgemm.FGEMM_EPI_ACT | fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr(),
            act=fgemm.FGEMM_ACT_GELU_TANH), beta=0.5)
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, (M, N, K)
        # RoPE with head width 8 and an offset
        _, Q, _ = oracle.gemm(A, B, beta=0.5, C=C, dtype=dtype, epi=oracle.EPI_ROPE,
                              rope_pos=np.arange(M) + 3, rope_head_dim=8)
        got = run_transform(A, B, C, dtype, fgemm.make_epilogue(
            fgemm.FGEMM_EPI_ROPE, rope_offset=3, rope_head_dim=8), beta=0.5)
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, (M, N, K)
        if N % 16:
            continue
        # SwiGLU backward with the row-scale gradient (op(B) is 2 * (N/2) wide)
        F = N // 2
        dO = inputs.normal((M, F), 785, dtype)
        ss = np.random.default_rng(786).uniform(1, 3, M).astype(np.float32)
        _, Qh, rgr = oracle.swiglu_bwd(A, B, dO, rms_ss=ss.astype(np.float64), rms_n=8,
                                       rms_eps=1e-6, dtype=dtype)
        Ad, Bd, dOd = to_dev(A, dtype), to_dev(B, dtype), to_dev(dO, dtype)
        ssd = torch.from_numpy(ss).cuda()
        rg = dev_f32(M)
        dH = empty_out(M, N, dtype)
        handle().gemm(Ad, Bd, dH, epilogue=fgemm.make_epilogue(
            fgemm.FGEMM_EPI_SWIGLU_BWD, rms_rowsumsq=ssd.data_ptr(), rms_n=8, rms_eps=1e-6,
            swiglu_dout=dOd.data_ptr(), swiglu_ldd=F, rms_grad=rg.data_ptr()))
        torch.cuda.synchronize()
        got = from_dev(dH)
        if K == 0:
            assert not np.any(oracle.decode(got, dtype)) and not np.any(rg.cpu().numpy())
        else:
            assert rel_err(got, Qh, dtype) <= CLASSICAL_TOL, (M, N, K)
            assert np.linalg.norm(rg.cpu().numpy() - rgr) <= STATS_TOL * np.linalg.norm(rgr)


def test_plan_cache_keeps_beta_and_epilogue_apart():
    """64 x 1024 x 16384 is a shape where the model splits K when there is no
    epilogue.  A call with beta != 0 and no epilogue, then one with SiLU and beta = 0,
    on one fresh handle: the second must get a plan of its own (the split-K path has
    no activation), and both must match the oracle."""
    import torch
    M, N, K, dtype = 64, 1024, 16384, BF16
    say(f"plan cache beta/epilogue {M}x{N}x{K}")
    A = inputs.normal((M, K), 731, dtype)
    B = inputs.normal((K, N), 732, dtype, std=0.02)
    C = inputs.normal((M, N), 733, dtype)
    _, Q1, _ = oracle.gemm(A, B, beta=0.5, C=C, dtype=dtype)
    _, Q2, _ = oracle.gemm(A, B, dtype=dtype, epi=oracle.EPI_ACT, act=oracle.ACT_SILU)
    h = fgemm.Handle(0)
    try:
        assert h.select(M, N, K).split_k > 1
        Ad, Bd, Cd = to_dev(A, dtype), to_dev(B, dtype), to_dev(C, dtype)
        h.gemm(Ad, Bd, Cd, beta=0.5)
        Od = empty_out(M, N, dtype)
        h.gemm(Ad, Bd, Od, epilogue=fgemm.make_epilogue(fgemm.FGEMM_EPI_ACT,
                                                          act=fgemm.FGEMM_ACT_SILU))
        torch.cuda.synchronize()
        assert rel_err(from_dev(Cd), Q1, dtype) <= CLASSICAL_TOL
        assert rel_err(from_dev(Od), Q2, dtype) <= CLASSICAL_TOL
    finally:
        h.close()


# ------------------------------------------------------------ A stored K x M (transA)
EPI_KINDS = ["bias_rowsumsq", "act", "rope", "rms_swiglu", "swiglu_bwd", "rms_bwd"]


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("tile", [(256, 256), (64, 128)])
@pytest.mark.parametrize("transB", [False, True])
@pytest.mark.parametrize("kind", EPI_KINDS)
def test_every_epilogue_with_transposed_a(dtype, tile, transB, kind):
    """Each epilogue kind with A stored K x M (the transposed-A load path has its own
    kernel instances), ragged M, against the oracle: output within 1e-3, row
    statistics and the row-scale gradient within 1e-3."""
    import torch
    M, K, N = 264, 192, 256  # N: output width (gate|up take 2N columns of op(B))
    say(f"transA epilogue {kind} dtype={dtype} tile={tile} tB={transB}")
    At = inputs.normal((K, M), 781, dtype)
    two = kind in ("rms_swiglu", "swiglu_bwd")
    W = inputs.normal((K, 2 * N if two else N), 782, dtype, std=0.1)
    Wst = np.ascontiguousarray(W.T) if transB else W
    Ad, Wd = to_dev(At, dtype), to_dev(Wst, dtype)
    plan = fgemm.classical_plan(*tile)
    ss = (np.random.default_rng(783).uniform(0.5, 2.0, M) * 4096).astype(np.float32)
    ssd = torch.from_numpy(ss).cuda()
    common = dict(transA=True, transB=transB, dtype=dtype)
    if kind == "swiglu_bwd":
        dO = inputs.normal((M, N), 784, dtype)
        dOd = to_dev(dO, dtype)
        rg = dev_f32(M)
        Cd = empty_out(M, 2 * N, dtype)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_SWIGLU_BWD, rms_rowsumsq=ssd.data_ptr(),
                                  rms_n=4096, rms_eps=1e-6, swiglu_dout=dOd.data_ptr(),
                                  swiglu_ldd=N, rms_grad=rg.data_ptr())
        handle().gemm(Ad, Wd, Cd, transA=True, transB=transB, alpha=1.5, epilogue=epi, plan=plan)
        torch.cuda.synchronize()
        _, Q, rgr = oracle.swiglu_bwd(At, Wst, dO, rms_ss=ss.astype(np.float64), rms_n=4096,
                                      alpha=1.5, **common)
        assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL
        got = rg.cpu().numpy().astype(np.float64)
        assert np.linalg.norm(got - rgr) <= STATS_TOL * np.linalg.norm(rgr)
        return
    if kind == "rms_bwd":
        X = inputs.normal((M, N), 785, dtype)
        rgrad = np.random.default_rng(786).normal(size=M).astype(np.float32)
        Xd, rgd = to_dev(X, dtype), torch.from_numpy(rgrad).cuda()
        Cd = empty_out(M, N, dtype)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_BWD, rms_rowsumsq=ssd.data_ptr(), rms_n=4096,
                                  rms_eps=1e-6, rms_grad=rgd.data_ptr(), rms_x=Xd.data_ptr(),
                                  rms_ldx=N)
        handle().gemm(Ad, Wd, Cd, transA=True, transB=transB, alpha=0.75, epilogue=epi, plan=plan)
        torch.cuda.synchronize()
        _, Q = oracle.rms_bwd(At, Wst, X, rms_ss=ss.astype(np.float64),
                              rgrad=rgrad.astype(np.float64), rms_n=4096, alpha=0.75, **common)
        assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL
        return
    C = inputs.normal((M, N), 787, dtype)
    bias = inputs.normal((N,), 788, dtype)
    Cd, bd = to_dev(C, dtype), to_dev(bias[None, :], dtype)
    ssout = dev_f32(M)
    pos = np.random.default_rng(789).integers(0, 4096, size=M).astype(np.int32)
    posd = torch.from_numpy(pos).cuda()
    if kind == "bias_rowsumsq":
        flags, oflags, extra = (fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ,
                                oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ, {})
        epi = fgemm.make_epilogue(flags, bias=bd.data_ptr(), rowsumsq=ssout.data_ptr())
    elif kind == "act":
        oflags, extra = oracle.EPI_BIAS | oracle.EPI_ACT, dict(act=oracle.ACT_GELU_TANH)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ACT, bias=bd.data_ptr(),
                                  act=fgemm.FGEMM_ACT_GELU_TANH)
    elif kind == "rope":
        oflags, extra = oracle.EPI_ROPE, dict(rope_pos=pos, rope_head_dim=64)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROPE, rope_positions=posd.data_ptr(),
                                  rope_head_dim=64, rope_theta=10000.0)
    else:  # rms_swiglu
        oflags, extra = oracle.EPI_RMS_SWIGLU, dict(rms_ss=ss.astype(np.float64), rms_n=4096)
        epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=ssd.data_ptr(),
                                  rms_n=4096, rms_eps=1e-6)
    _, Q, ssr = oracle.gemm(At, Wst, alpha=1.25, beta=0.5, C=C, epi=oflags,
                            bias=bias if oflags & oracle.EPI_BIAS else None, **extra, **common)
    handle().gemm(Ad, Wd, Cd, transA=True, transB=transB, alpha=1.25, beta=0.5, epilogue=epi,
                  plan=plan)
    torch.cuda.synchronize()
    assert rel_err(from_dev(Cd), Q, dtype) <= CLASSICAL_TOL
    if kind == "bias_rowsumsq":
        got = ssout.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - ssr) / ssr) <= STATS_TOL
