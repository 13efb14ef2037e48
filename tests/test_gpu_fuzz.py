"""Seeded shape fuzz of the classical path: M, N, K drawn from 1..600, every layout,
both 16-bit types, padded leading dimensions, alpha/beta/bias, through the
library's own plan and through a forced tile.

Integer inputs: every product, sum, alpha*acc, beta*C and bias term is an integer
(or a half) far below 2^24, so the kernel's fp32 value is the exact one and its
round-to-nearest-even 16-bit output must equal the oracle's rounding of the exact
fp64 result bit for bit.  Padding columns hold NaN bits, so a read past the
logical edge shows in the output.  Normal-valued cases are held to the
elementwise fp32 summation bound of the oracle."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import BF16, F16, check_full, from_dev, handle, run, say, to_dev

pytestmark = pytest.mark.gpu

TILES = [(256, 256), (128, 128), (64, 128), (32, 128), (64, 64)]
ALPHAS = [1.0, -1.0, 2.0]
BETAS = [0.0, 0.5, 1.0]


def draw_dim(rng):
    """1..600, with extra weight on the tile and chunk boundaries (x*8 - 1 .. x*8 + 1)
    and on the degenerate 1."""
    r = rng.random()
    if r < 0.1:
        return 1
    if r < 0.4:
        base = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
        return int(np.clip(base + rng.integers(-1, 2), 1, 600))
    return int(rng.integers(1, 601))


def cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(
            M=draw_dim(rng), N=draw_dim(rng), K=draw_dim(rng),
            transA=bool(rng.integers(2)), transB=bool(rng.integers(2)),
            dtype=BF16 if rng.integers(2) else F16,
            pad=tuple(int(p) for p in rng.choice([0, 0, 1, 3, 8], size=3)),
            alpha=float(rng.choice(ALPHAS)), beta=float(rng.choice(BETAS)),
            bias=bool(rng.random() < 0.3),
            tile=TILES[int(rng.integers(len(TILES)))],
            seed=1000 + 7 * i))
    return out


def operands(c, kind):
    M, N, K, dt = c["M"], c["N"], c["K"], c["dtype"]
    shapeA = (K, M) if c["transA"] else (M, K)
    shapeB = (N, K) if c["transB"] else (K, N)
    if kind == "int":
        lo = -1 if dt == BF16 else -2
        A = inputs.integers(shapeA, c["seed"], dt, lo, -lo)
        B = inputs.integers(shapeB, c["seed"] + 1, dt, lo, -lo)
        C = inputs.integers((M, N), c["seed"] + 2, dt, -4, 4)
        bias = inputs.integers((N,), c["seed"] + 3, dt, -3, 3)
    else:
        A = inputs.normal(shapeA, c["seed"], dt)
        B = inputs.normal(shapeB, c["seed"] + 1, dt)
        C = inputs.normal((M, N), c["seed"] + 2, dt)
        bias = inputs.normal((N,), c["seed"] + 3, dt)
    return A, B, C, bias


def run_case(c, A, B, C, bias, plan):
    """The device result of one case (bias through the BIAS epilogue)."""
    dt = c["dtype"]
    if not c["bias"]:
        return run(A, B, dt, transA=c["transA"], transB=c["transB"], alpha=c["alpha"],
                   beta=c["beta"], C_bits=C if c["beta"] != 0.0 else None, pad=c["pad"],
                   plan=plan)
    import torch
    pa, pb, pc = c["pad"]
    Ad, Bd = to_dev(A, dt, pa), to_dev(B, dt, pb)
    Cin = C if c["beta"] != 0.0 else np.full(C.shape, 0x7FC0, dtype=np.uint16)
    Cd = to_dev(Cin, dt, pc)
    bd = to_dev(bias[None, :], dt)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS, bias=bd.data_ptr())
    handle().gemm(Ad, Bd, Cd, transA=c["transA"], transB=c["transB"], alpha=c["alpha"],
                  beta=c["beta"], plan=plan, epilogue=epi)
    torch.cuda.synchronize()
    return from_dev(Cd)


def reference(c, A, B, C, bias):
    kw = dict(transA=c["transA"], transB=c["transB"], alpha=c["alpha"], beta=c["beta"],
              C=C if c["beta"] != 0.0 else None, dtype=c["dtype"])
    if c["bias"]:
        kw.update(epi=oracle.EPI_BIAS, bias=bias)
    return kw


def unsigned_zero(bits):
    """16-bit patterns with -0 written as +0: an exact zero's sign depends on the
    order in which zero terms are added, which is not part of the product."""
    bits = np.asarray(bits, dtype=np.uint16).ravel().copy()
    bits[bits == 0x8000] = 0
    return bits


def name(c):
    return (f"M={c['M']} N={c['N']} K={c['K']} tA={int(c['transA'])} tB={int(c['transB'])} "
            f"dtype={c['dtype']} pad={c['pad']} alpha={c['alpha']} beta={c['beta']} "
            f"bias={int(c['bias'])} tile={c['tile']}")


@pytest.mark.parametrize("block", range(4))
def test_fuzz_exact_integers(block):
    for c in cases(4242 + block, 16):
        A, B, C, bias = operands(c, "int")
        _, Q, _ = oracle.gemm(A, B, **reference(c, A, B, C, bias))
        for plan, label in ((None, "auto"), (fgemm.classical_plan(*c["tile"]), "tile")):
            say(f"fuzz exact {label} {name(c)}")
            got = run_case(c, A, B, C, bias, plan)
            bad = np.flatnonzero(unsigned_zero(got) != unsigned_zero(Q))
            assert bad.size == 0, (label, name(c), bad[:8])


@pytest.mark.parametrize("block", range(2))
def test_fuzz_random_elementwise_bound(block):
    """Every output within the fp32 summation bound plus the 16-bit rounding; the
    normwise 1e-3 figure only where the output is large enough for it to be an
    average (one legitimate 1-ulp rounding flip of a 1 x 1 output is 2^-8)."""
    for c in cases(9191 + block, 12):
        A, B, C, bias = operands(c, "normal")
        kw = reference(c, A, B, C, bias)
        kw.pop("epi", None), kw.pop("bias", None)
        D, S = oracle.gemm_dense(A, B, bound=True, **kw)
        if c["bias"]:
            bv = oracle.decode(bias, c["dtype"])
            D, S = D + bv[None, :], S + np.abs(bv)[None, :]
        for plan, label in ((None, "auto"), (fgemm.classical_plan(*c["tile"]), "tile")):
            say(f"fuzz random {label} {name(c)}")
            got = run_case(c, A, B, C, bias, plan)
            if D.size >= 65536:
                check_full(got, D, S, c["K"], c["dtype"])
            else:
                g = oracle.decode(got, c["dtype"])
                bad = ~(np.abs(g - D) <= oracle.elementwise_bound(D, S, c["K"], c["dtype"]))
                assert not bad.any(), (label, name(c), np.argwhere(bad)[:4])
