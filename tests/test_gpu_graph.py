"""fgemm_gemm under HIP graph capture (torch.cuda.graph): once a first eager call
per shape has sized the handle's workspace, a call enqueues kernels only (no
allocation, no memset, no synchronisation), so it can be captured.  Each replay
must reproduce the eager result bit for bit (the kernels are deterministic); eager
work and synchronisations run between the replays."""
import numpy as np
import pytest

import oracle
from hgemm_strassen_type_amd import fgemm
from hgemm_strassen_type_amd import inputs
from gpu_util import BF16, F16, CLASSICAL_TOL, STRASSEN_TOL, from_dev, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    say("graph capture: classical+bias+rowsumsq, split-K, winograd d1")
    h = fgemm.Handle(0)
    try:
        # classical with bias and row statistics (bf16), ragged
        A1 = to_dev(inputs.normal((520, 384), 801, BF16), BF16)
        B1 = to_dev(inputs.normal((384, 392), 802, BF16, std=0.1), BF16)
        bias = to_dev(inputs.normal((392,), 803, BF16)[None, :], BF16)
        C1 = torch.empty((520, 392), dtype=torch.bfloat16, device="cuda")
        ss = torch.empty(520, dtype=torch.float32, device="cuda")
        e1 = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS | fgemm.FGEMM_EPI_ROWSUMSQ,
                                 bias=bias.data_ptr(), rowsumsq=ss.data_ptr())
        # split K on a decode-like shape (fp32 slices + finalize)
        A2 = to_dev(inputs.normal((16, 2048), 804, BF16), BF16)
        B2 = to_dev(inputs.normal((2048, 1024), 805, BF16, std=0.02), BF16)
        C2 = torch.empty((16, 1024), dtype=torch.bfloat16, device="cuda")
        p2 = fgemm.classical_plan(32, 128, split_k=4)
        # Winograd depth 1 (fp16): max|x|, scales, pre-adds, batched products, post-add
        A3b = inputs.uniform((512, 512), 806, F16)
        B3b = inputs.uniform((512, 512), 807, F16)
        A3, B3 = to_dev(A3b, F16), to_dev(B3b, F16)
        C3 = torch.empty((512, 512), dtype=torch.float16, device="cuda")
        p3 = fgemm.strassen_plan(1, fgemm.FGEMM_VARIANT_WINOGRAD)

        def calls():
            h.gemm(A1, B1, C1, alpha=1.25, epilogue=e1)
            h.gemm(A2, B2, C2, plan=p2)
            h.gemm(A3, B3, C3, plan=p3)

        calls()  # eager: sizes the workspace
        torch.cuda.synchronize()
        ref = [from_dev(C1), ss.cpu().numpy().copy(), from_dev(C2), from_dev(C3)]
        # the eager results themselves against the oracle
        _, Q3, _ = oracle.gemm(A3b, B3b, dtype=F16)
        assert rel_err(ref[3], Q3, F16) <= STRASSEN_TOL
        _, Q2, _ = oracle.gemm(from_dev(A2), from_dev(B2), dtype=BF16)
        assert rel_err(ref[2], Q2, BF16) <= CLASSICAL_TOL

        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            calls()  # warm the side stream too
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            calls()
        torch.cuda.synchronize()
        for r in range(3):
            # eager work between replays: scribble over every output
            for t in (C1, C2, C3):
                t.fill_(float("nan"))
            ss.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = [from_dev(C1), ss.cpu().numpy(), from_dev(C2), from_dev(C3)]
            for i, (a, b) in enumerate(zip(got, ref)):
                assert np.array_equal(a, b), (r, i)
        del g
    finally:
        h.close()


def test_graph_quantize_then_low_precision_gemms():
    """The MX quantizer (row-wise and transposed) feeding the MXFP4 and MXFP8 GEMMs,
    captured in one graph: neither allocates nor synchronises, so every replay
    reproduces the eager codes, scales and products bit for bit."""
    import torch
    say("graph capture: quantize_mx + mxf4 + mxf8 chain")
    h = fgemm.Handle(0)
    try:
        M, N, K = 512, 384, 1024
        X = to_dev(inputs.normal((M, K), 811, BF16), BF16)
        W = to_dev(inputs.normal((K, N), 812, BF16, std=0.02), BF16)
        E4, E2 = fgemm.FGEMM_E4M3, fgemm.FGEMM_E2M1
        qx4, sx4 = fgemm.quantize_mx(X, E2)
        qw4, sw4 = fgemm.quantize_mx(W, E2, transpose=True)
        qx8, sx8 = fgemm.quantize_mx(X, E4)
        qw8, sw8 = fgemm.quantize_mx(W, E4, transpose=True)
        C4 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        C8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def calls():
            fgemm.quantize_mx(X, E2, Q=qx4, scales=sx4)
            fgemm.quantize_mx(W, E2, transpose=True, Q=qw4, scales=sw4)
            fgemm.quantize_mx(X, E4, Q=qx8, scales=sx8)
            fgemm.quantize_mx(W, E4, transpose=True, Q=qw8, scales=sw8)
            h.gemm_mxf4(qx4, qw4, C4, sx4, sw4)
            h.gemm_mxf8(qx8, qw8, C8, sx8, sw8)

        calls()
        torch.cuda.synchronize()
        outs = (qx4, sx4, qw4, sw4, qx8, sx8, qw8, sw8)
        ref = [t.cpu().numpy().copy() for t in outs] + [from_dev(C4), from_dev(C8)]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            calls()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            calls()
        torch.cuda.synchronize()
        for r in range(3):
            for t in (qx4, qw4, qx8, qw8):
                t.fill_(0xAA)
            for t in (sx4, sw4, sx8, sw8):   # the written scale columns (K/32 a row)
                t[:, :K // 32].fill_(0xAA)
            C4.fill_(float("nan"))
            C8.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = [t.cpu().numpy() for t in outs] + [from_dev(C4), from_dev(C8)]
            for i, (a, b) in enumerate(zip(got, ref)):
                assert np.array_equal(a, b), (r, i)
        del g
    finally:
        h.close()
