"""fgemm_gemm_noalloc, the entry point for callers that cannot allocate device memory,
through the C ABI: on the same inputs it must give the bits fgemm_gemm gives (the
same classical plan and kernels, its scratch in the fixed device array instead of
the handle's workspace), and both must be within the oracle's tolerances.  Calls
come in a row: a split-K problem (fp32 slices in the scratch), then a smaller
problem with row statistics (per-wave partials in the scratch), then the first
again over the second's leftovers.  A call whose plan needs more scratch than the
array holds is refused before anything is enqueued."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import BF16, CLASSICAL_TOL, STATS_TOL, from_dev, handle, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _call(noalloc, A, B, C_bits, dtype, *, alpha, beta, bias=None, stats=False):
    import torch
    Cd = to_dev(C_bits, dtype)
    flags = 0
    kw = {}
    if bias is not None:
        flags |= fgemm.FGEMM_EPI_BIAS
        kw["bias"] = bias.data_ptr()
    ssd = None
    if stats:
        ssd = torch.full((Cd.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
        flags |= fgemm.FGEMM_EPI_ROWSUMSQ
        kw["rowsumsq"] = ssd.data_ptr()
    epi = fgemm.make_epilogue(flags, **kw) if flags else None
    handle().gemm(A, B, Cd, alpha=alpha, beta=beta, epilogue=epi, noalloc=noalloc)
    torch.cuda.synchronize()
    return from_dev(Cd), (ssd.cpu().numpy() if stats else None)


def test_noalloc_matches_fgemm_gemm_on_calls_in_a_row():
    import torch
    dtype = BF16
    h = handle()
    # 1: a decode-like skinny shape that the model splits over K
    M1, N1, K1 = 64, 1024, 16384
    assert h.select(M1, N1, K1).split_k > 1
    A1, B1 = inputs.normal((M1, K1), 701, dtype), inputs.normal((K1, N1), 702, dtype, std=0.02)
    C1 = inputs.normal((M1, N1), 703, dtype)
    bias1 = inputs.normal((N1,), 704, dtype)
    _, Q1, _ = oracle.gemm(A1, B1, alpha=1.25, beta=0.5, C=C1, dtype=dtype, epi=oracle.EPI_BIAS,
                           bias=bias1)
    # 2: smaller, with row statistics
    M2, N2, K2 = 300, 200, 256
    A2, B2 = inputs.normal((M2, K2), 711, dtype), inputs.normal((K2, N2), 712, dtype)
    C2 = inputs.normal((M2, N2), 713, dtype)
    bias2 = inputs.normal((N2,), 714, dtype)
    _, Q2, ss2 = oracle.gemm(A2, B2, alpha=0.75, beta=-0.5, C=C2, dtype=dtype,
                             epi=oracle.EPI_BIAS | oracle.EPI_ROWSUMSQ, bias=bias2)
    d1 = [to_dev(A1, dtype), to_dev(B1, dtype), to_dev(bias1[None, :], dtype)]
    d2 = [to_dev(A2, dtype), to_dev(B2, dtype), to_dev(bias2[None, :], dtype)]
    for step, (d, C, Q, ss, kw) in enumerate([
            (d1, C1, Q1, None, dict(alpha=1.25, beta=0.5)),
            (d2, C2, Q2, ss2, dict(alpha=0.75, beta=-0.5, stats=True)),
            (d1, C1, Q1, None, dict(alpha=1.25, beta=0.5))]):
        say(f"noalloc call {step}: {d[0].shape[0]}x{d[1].shape[1]}x{d[0].shape[1]}")
        got, ss_got = _call(True, d[0], d[1], C, dtype, bias=d[2][0], **kw)
        ref, ss_ref = _call(False, d[0], d[1], C, dtype, bias=d[2][0], **kw)
        assert np.array_equal(got, ref), step
        assert rel_err(got, Q, dtype) <= CLASSICAL_TOL, step
        if ss is not None:
            assert np.array_equal(ss_got, ss_ref), step
            assert np.max(np.abs(ss_got - ss) / ss) <= STATS_TOL, step
    torch.cuda.synchronize()


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    """Row statistics of 32800 rows over 65536 columns need 256-column tiles x 2
    wave columns x 32800 rows of fp32 partials, 67 MB, above the 64 MiB array: the
    call returns FGEMM_ERR_WORKSPACE and enqueues nothing (the output keeps its
    values).  fgemm_gemm takes the same call through the handle's workspace."""
    import torch
    say("noalloc refusal")
    M, N, K = 32800, 65536, 8
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    ssd = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=ssd.data_ptr())
    h = handle()
    assert h.select(M, N, K, epilogue=epi).workspace_bytes > fgemm.FGEMM_NOALLOC_SCRATCH_BYTES
    st = fgemm.fgemm_gemm_noalloc(h.h, 0, 0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0,
                                  C.data_ptr(), N, fgemm.FGEMM_BF16, epi, fgemm.current_stream(),
                                  check=False)
    assert st == fgemm.FGEMM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((C[::997, ::991] == 3.0).all()) and bool((ssd == -1.0).all())
    h.gemm(A, B, C, epilogue=epi)
    torch.cuda.synchronize()
    assert bool((C[::997, ::991] == 0.0).all()) and bool((ssd == 0.0).all())
    del A, B, C, ssd
    torch.cuda.empty_cache()
