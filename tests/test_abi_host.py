"""CPU tests of the C ABI: the library loads and exports every declared symbol,
argument validation, the quantization helpers against the worked examples of the
CS336 Lecture 05 notes (Pages 43 and 48), and the decision model's properties."""
import ctypes
import os
import re

import pytest

from hgemm_strassen_type_amd import fgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N_, T_ = fgemm.FGEMM_OP_N, fgemm.FGEMM_OP_T
BF, HF = fgemm.FGEMM_BF16, fgemm.FGEMM_F16
OK, INVAL, NOTSUP = fgemm.FGEMM_OK, fgemm.FGEMM_ERR_INVALID_VALUE, fgemm.FGEMM_ERR_NOT_SUPPORTED


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fgemm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = fgemm.lib()
    names = declared_functions()
    assert set(names) == set(fgemm.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    assert fgemm.status_name(OK) == "FGEMM_OK"
    assert fgemm.status_name(fgemm.FGEMM_ERR_WORKSPACE) == "FGEMM_ERR_WORKSPACE"
    assert fgemm.status_name(77) == "FGEMM_UNKNOWN_STATUS"


# ---------------------------------------------------------------- quantization
def test_tile_quantization_page_example():
    # 256 / 128 -> 2 tiles per dimension, 257 / 128 -> 3
    assert fgemm.fgemm_tile_count(256, 256, 128, 128) == 4
    assert fgemm.fgemm_tile_count(257, 257, 128, 128) == 9
    assert fgemm.fgemm_tile_count(256, 1, 128, 128) == 2
    assert fgemm.fgemm_tile_count(257, 1, 128, 128) == 3


def test_wave_quantization_page_example():
    # N = 1792 with 256x128 tiles: 7 x 14 = 98 tiles, one wave on 108 units
    tiles = fgemm.fgemm_tile_count(1792, 1792, 256, 128)
    assert tiles == 98
    waves, tail = fgemm.fgemm_wave_count(tiles, 108)
    assert waves == 1 and tail == pytest.approx(98 / 108)
    # N = 1793: 8 x 15 = 120 tiles, two waves, the second 12/108 busy
    tiles = fgemm.fgemm_tile_count(1793, 1793, 256, 128)
    assert tiles == 120
    waves, tail = fgemm.fgemm_wave_count(tiles, 108)
    assert waves == 2 and tail == pytest.approx(12 / 108)
    assert round(tail * 100, 1) == 11.1


def test_quantization_rejects_bad_input():
    assert fgemm.fgemm_tile_count(-1, 4, 1, 1) == -1
    assert fgemm.fgemm_tile_count(4, 4, 0, 1) == -1
    assert fgemm.fgemm_wave_count(4, 0)[0] == -1


# ------------------------------------------------------------ argument checks
P = 0x10000  # a fake non-null device address (never dereferenced by the check)


def chk(ta=N_, tb=N_, M=64, N=64, K=64, A=P, lda=None, B=P, ldb=None, beta=0.0, C=P, ldc=None,
        dtype=BF, epi=None):
    if lda is None:
        lda = K if ta == N_ else M
    if ldb is None:
        pair = fgemm.FGEMM_EPI_RMS_SWIGLU | fgemm.FGEMM_EPI_SWIGLU_BWD
        nb = 2 * N if epi is not None and epi.flags & pair else N
        ldb = nb if tb == N_ else K
    if ldc is None:
        ldc = N
    return fgemm.fgemm_check_args(ta, tb, M, N, K, A, lda, B, ldb, beta, C, ldc, dtype, epi)


def test_check_args_accepts_valid_calls():
    assert chk() == OK
    for ta in (N_, T_):
        for tb in (N_, T_):
            assert chk(ta=ta, tb=tb, M=33, N=17, K=9) == OK
    assert chk(M=0, A=None, B=None, C=None) == OK          # nothing to do
    assert chk(K=0, A=None, B=None, lda=1) == OK           # C = beta*C
    assert chk(dtype=HF) == OK


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(lda=63), dict(ldb=63), dict(ldc=63),
    dict(ta=2), dict(tb=-1), dict(dtype=3),
    dict(A=None), dict(B=None), dict(C=None),
    dict(ta=T_, lda=63),                                     # A stored K x M: lda >= M
    dict(tb=T_, ldb=63),                                     # B stored N x K: ldb >= K
])
def test_check_args_rejects(kw):
    assert chk(**kw) == INVAL


def test_check_args_epilogues():
    E = fgemm.make_epilogue
    assert chk(epi=E(fgemm.FGEMM_EPI_BIAS, bias=P)) == OK
    assert chk(epi=E(fgemm.FGEMM_EPI_BIAS)) == INVAL                      # no bias pointer
    assert chk(epi=E(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=P)) == OK
    assert chk(epi=E(fgemm.FGEMM_EPI_ROWSUMSQ)) == INVAL
    sw = E(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=P, rms_n=4096, rms_eps=1e-6)
    assert chk(epi=sw) == OK
    assert chk(epi=sw, ldb=64) == INVAL                                    # B needs 2N columns
    assert chk(epi=E(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=P, rms_n=0)) == INVAL
    assert chk(epi=E(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_n=4096)) == INVAL     # no statistics
    assert chk(epi=E(fgemm.FGEMM_EPI_RMS_SWIGLU | fgemm.FGEMM_EPI_BIAS, bias=P, rms_rowsumsq=P,
                     rms_n=4096)) == NOTSUP
    assert chk(epi=E(64)) == INVAL                                         # unknown flag
    # activation and rotary embedding: one of them, with bias and statistics
    ACT, ROPE = fgemm.FGEMM_EPI_ACT, fgemm.FGEMM_EPI_ROPE
    for a in (fgemm.FGEMM_ACT_RELU, fgemm.FGEMM_ACT_SILU, fgemm.FGEMM_ACT_GELU_TANH):
        assert chk(epi=E(ACT | fgemm.FGEMM_EPI_BIAS, bias=P, act=a)) == OK
    assert chk(epi=E(ACT, act=0)) == INVAL
    assert chk(epi=E(ACT, act=4)) == INVAL
    assert chk(epi=E(ROPE | fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=P, rope_head_dim=16)) == OK
    assert chk(epi=E(ROPE, rope_positions=P, rope_head_dim=64)) == OK
    assert chk(epi=E(ROPE, rope_head_dim=0)) == INVAL
    assert chk(epi=E(ROPE, rope_head_dim=7)) == INVAL                      # odd
    assert chk(epi=E(ROPE, rope_head_dim=48)) == INVAL                     # does not divide N
    assert chk(epi=E(ROPE, rope_head_dim=16, rope_theta=0.0)) == INVAL
    assert chk(epi=E(ROPE, rope_head_dim=4)) == NOTSUP                     # kernels: hd % 8 == 0
    assert chk(N=2048, epi=E(ROPE, rope_head_dim=2048)) == NOTSUP           # table of 512 pairs
    assert chk(epi=E(ACT | ROPE, act=1, rope_head_dim=16)) == NOTSUP
    assert chk(epi=E(fgemm.FGEMM_EPI_RMS_SWIGLU | ACT, rms_rowsumsq=P, rms_n=4096,
                     act=1)) == NOTSUP
    # SwiGLU backward: 2N-wide output, the incoming gradient, beta 0, alone
    BWD = fgemm.FGEMM_EPI_SWIGLU_BWD
    bw = E(BWD, rms_rowsumsq=P, rms_n=4096, rms_eps=1e-6, swiglu_dout=P, swiglu_ldd=64)
    assert chk(epi=bw, ldc=128) == OK
    assert chk(epi=bw, ldc=64) == INVAL                                    # output is 2N wide
    assert chk(epi=bw, ldc=128, beta=0.5) == NOTSUP
    assert chk(epi=E(BWD, rms_rowsumsq=P, rms_n=4096, swiglu_ldd=64), ldc=128) == INVAL  # no dO
    assert chk(epi=E(BWD, rms_rowsumsq=P, rms_n=4096, swiglu_dout=P, swiglu_ldd=32), ldc=128) == INVAL
    assert chk(epi=E(BWD | fgemm.FGEMM_EPI_BIAS, bias=P, rms_rowsumsq=P, rms_n=4096,
                     swiglu_dout=P, swiglu_ldd=64), ldc=128) == NOTSUP
    assert chk(epi=E(BWD | fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=P, rms_n=4096,
                     swiglu_dout=P, swiglu_ldd=64), ldc=128) == NOTSUP
    # RMS backward: alone, beta 0, the input X, the scale gradient and the statistics
    RB = fgemm.FGEMM_EPI_RMS_BWD
    rb = dict(rms_rowsumsq=P, rms_n=4096, rms_eps=1e-6, rms_grad=P, rms_x=P, rms_ldx=64)
    assert chk(epi=E(RB, **rb)) == OK
    assert chk(epi=E(RB, **rb), beta=1.0) == NOTSUP
    assert chk(epi=E(RB | fgemm.FGEMM_EPI_BIAS, bias=P, **rb)) == NOTSUP
    assert chk(epi=E(RB, **{**rb, "rms_x": 0})) == INVAL
    assert chk(epi=E(RB, **{**rb, "rms_grad": 0})) == INVAL
    assert chk(epi=E(RB, **{**rb, "rms_ldx": 32})) == INVAL
    assert chk(epi=E(RB, **{**rb, "rms_n": 0})) == INVAL


# ---------------------------------------------------------------- decision model
def mi355x_model(**over):
    m = fgemm.fgemm_model_t()
    m.compute_units, m.peak_tflops, m.hbm_gbps = 256, 256 * 4096 * 2.4e9 / 1e12, 8000.0
    m.eta_mfma, m.eta_hbm, m.launch_us, m.max_workspace_bytes = 0.7, 0.8, 4.0, 16 * 2.0 ** 30
    m.max_rel_err = 5e-3
    for k, v in over.items():
        setattr(m, k, v)
    return m


def select(M, N, K, model=None, epi=None, dtype=BF):
    return fgemm.fgemm_select_model(model or mi355x_model(), N_, N_, M, N, K, dtype, epi)


def test_select_never_picks_strassen_where_it_cannot_run():
    for shape in [(1, 14336, 4096), (16, 14336, 4096), (64, 14336, 4096), (8191, 8192, 8192),
                  (256, 256, 256), (8192, 8192, 8200)]:
        assert select(*shape).path == fgemm.FGEMM_PATH_CLASSICAL, shape
    # SwiGLU: the recursion runs on op(B)'s 2N columns, which must divide by 8*2^depth
    fast_mem = mi355x_model(hbm_gbps=80000.0)
    epi = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=P, rms_n=4096,
                              rms_eps=1e-6)
    assert select(16384, 16380, 16384, fast_mem, epi=epi).path == fgemm.FGEMM_PATH_CLASSICAL


def test_select_strassen_with_epilogues():
    # every epilogue runs in the Strassen post-add: where the multiply saving wins,
    # the bias and RMS + SwiGLU epilogues take the Strassen path too
    fast_mem = mi355x_model(hbm_gbps=80000.0)
    base = select(16384, 16384, 16384, fast_mem)
    bias = fgemm.make_epilogue(fgemm.FGEMM_EPI_BIAS, bias=P)
    p = select(16384, 16384, 16384, fast_mem, epi=bias)
    assert p.path == fgemm.FGEMM_PATH_STRASSEN
    assert p.workspace_bytes == base.workspace_bytes
    sw = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=P, rms_n=4096, rms_eps=1e-6)
    p = select(16384, 8192, 16384, fast_mem, epi=sw)
    assert p.path == fgemm.FGEMM_PATH_STRASSEN
    assert p.workspace_bytes == base.workspace_bytes  # op(B) is 16384 wide
    # on the MI355X constants the configured fused chain stays classical
    ss = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=P)
    for (M, N, K, e) in [(8192, 4096, 4096, ss), (8192, 11008, 4096, sw)]:
        assert select(M, N, K, epi=e).path == fgemm.FGEMM_PATH_CLASSICAL


def test_select_statistics_guard_keeps_row_sums_within_1e3():
    """A row's sum of squares of the written output moves by up to 2e + e^2 for an
    output relative error e, so row statistics (ROWSUMSQ) go to Strassen only where
    twice the plan's predicted error is within 1e-3.  No Strassen figure is that low,
    so every automatic ROWSUMSQ plan is classical, also where Strassen wins without
    statistics: with bandwidth to spare, and at 49152^3 and 65536^3 under the
    calibrated MI355X constants."""
    ss = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ, rowsumsq=P)
    ssb = fgemm.make_epilogue(fgemm.FGEMM_EPI_ROWSUMSQ | fgemm.FGEMM_EPI_BIAS, rowsumsq=P, bias=P)
    fast_mem = mi355x_model(hbm_gbps=80000.0)
    cal = mi355x_model(eta_mfma=0.52, eta_hbm=0.66, max_workspace_bytes=288e9 / 3)
    for (n, md) in [(16384, fast_mem), (49152, cal), (65536, cal)]:
        for dt in (BF, HF):
            assert select(n, n, n, md, dtype=dt).path == fgemm.FGEMM_PATH_STRASSEN, (n, dt)
            for e in (ss, ssb):
                p = select(n, n, n, md, epi=e, dtype=dt)
                assert p.path == fgemm.FGEMM_PATH_CLASSICAL, (n, dt)
                assert 2 * p.pred_rel_err <= 1e-3
    for dt in (BF, HF):
        for v in (fgemm.FGEMM_VARIANT_S69, fgemm.FGEMM_VARIANT_WINOGRAD):
            for d in (1, 2):
                assert 2 * fgemm.fgemm_plan_rel_err(dt, fgemm.strassen_plan(d, v)) > 1e-3


def test_select_predicted_time_is_monotone():
    prev = 0.0
    for n in (512, 1024, 2048, 4096, 8192, 16384):
        t = select(n, n, n).t_classical_pred_us
        assert t > prev
        prev = t
    assert select(8192, 8192, 8192).t_classical_pred_us < select(8192, 8192, 16384).t_classical_pred_us


def test_select_roofline_bounds():
    md = mi355x_model()
    n = 8192
    p = select(n, n, n, md)
    flops = 2.0 * n ** 3
    # never faster than the MFMA peak (roofline: min of peak and intensity x bandwidth)
    assert p.t_classical_pred_us * 1e-6 >= flops / (md.peak_tflops * 1e12)
    # decode: bandwidth term dominates, time >= weight bytes / bandwidth
    p = select(1, 14336, 4096, md)
    assert p.t_classical_pred_us * 1e-6 >= 4096 * 14336 * 2 / (md.hbm_gbps * 1e9)


def test_select_takes_strassen_when_compute_is_slow_relative_to_memory():
    # A machine with abundant bandwidth: the 7/8 multiply saving wins at large sizes.
    fast_mem = mi355x_model(hbm_gbps=80000.0)
    p = select(16384, 16384, 16384, fast_mem)
    assert p.path == fgemm.FGEMM_PATH_STRASSEN
    assert p.t_pred_us < p.t_classical_pred_us
    assert p.workspace_bytes > 0
    # Starved bandwidth: the addition traffic makes Strassen lose.
    slow_mem = mi355x_model(hbm_gbps=800.0)
    assert select(16384, 16384, 16384, slow_mem).path == fgemm.FGEMM_PATH_CLASSICAL
    # A workspace cap below the need keeps it classical.
    capped = mi355x_model(hbm_gbps=80000.0, max_workspace_bytes=1e6)
    assert select(16384, 16384, 16384, capped).path == fgemm.FGEMM_PATH_CLASSICAL


def test_select_tile_choice_follows_wave_quantization():
    # 256 output tiles of 256x256 fill exactly one wave on 256 units
    p = select(4096, 4096, 4096)
    assert (p.tile_m, p.tile_n) == (256, 256)
    # a single 256x256 tile would leave 255 units idle: smaller tiles win
    p = select(256, 256, 4096)
    assert p.tile_m * p.tile_n < 256 * 256
    # skinny M uses a skinny tile
    assert select(16, 14336, 4096).tile_m <= 64


def test_select_one_row_decode_tile():
    # the 64x64 tile is offered only while M fits one tile row; on the decode shapes
    # it ties with 32x128 in the model and wins the tie (one tile row, more tiles)
    for m in (1, 16, 64):
        p = select(m, 14336, 4096)
        assert (p.tile_m, p.tile_n, p.split_k) == (64, 64, 1), m
    for m in (65, 128, 1000):
        p = select(m, 14336, 4096)
        assert (p.tile_m, p.tile_n) != (64, 64), m
    # the SwiGLU epilogue needs both column halves in one wave: never the 64x64 tile
    e = fgemm.make_epilogue(fgemm.FGEMM_EPI_RMS_SWIGLU, rms_rowsumsq=1, rms_n=4096)
    p = select(16, 14336, 4096, epi=e)
    assert (p.tile_m, p.tile_n) not in ((64, 64), (32, 128))


def test_select_error_budget_sets_the_depth():
    """The accuracy guard: with bandwidth to spare (the multiply saving wins), the
    calibrated error of each variant and depth against the error budget decides how
    deep AUTO goes; a budget below every Strassen figure keeps the classical path."""
    def pick(budget, dtype):
        p = select(16384, 16384, 16384, mi355x_model(hbm_gbps=80000.0, max_rel_err=budget),
                   dtype=dtype)
        return p.path, p.depth, p.variant, p.pred_rel_err
    # default budget (the Strassen tolerance): the deepest, fastest candidate
    path, depth, variant, err = pick(5e-3, BF)
    assert (path, depth) == (fgemm.FGEMM_PATH_STRASSEN, 2) and err <= 5e-3
    # bf16 figures: S69 d1 < Winograd d1 < S69 d2 < Winograd d2
    path, depth, variant, err = pick(2e-3, BF)
    assert (path, depth, variant) == (fgemm.FGEMM_PATH_STRASSEN, 2, fgemm.FGEMM_VARIANT_S69)
    path, depth, variant, err = pick(1.5e-3, BF)
    assert (path, depth) == (fgemm.FGEMM_PATH_STRASSEN, 1) and err <= 1.5e-3
    path, depth, variant, err = pick(1e-3, BF)
    assert (path, depth, variant) == (fgemm.FGEMM_PATH_STRASSEN, 1, fgemm.FGEMM_VARIANT_S69)
    path, depth, variant, err = pick(5e-4, BF)
    assert path == fgemm.FGEMM_PATH_CLASSICAL and err <= 5e-4
    # fp16 carries less error through the same fp16 temporaries: 1e-3 still allows
    # Winograd at depth 1
    path, depth, variant, err = pick(1e-3, HF)
    assert (path, depth) == (fgemm.FGEMM_PATH_STRASSEN, 1) and err <= 1e-3
    # a model without a budget is refused
    m = mi355x_model()
    m.max_rel_err = 0.0
    with pytest.raises(fgemm.FgemmError):
        fgemm.fgemm_select_model(m, N_, N_, 1024, 1024, 1024, BF, None)


def test_plan_rel_err_model():
    cl = fgemm.classical_plan()
    assert 0 < fgemm.fgemm_plan_rel_err(BF, cl) <= 1e-4
    figs = {}
    for dt in (BF, HF):
        for v in (fgemm.FGEMM_VARIANT_S69, fgemm.FGEMM_VARIANT_WINOGRAD):
            for d in (1, 2):
                figs[dt, v, d] = fgemm.fgemm_plan_rel_err(dt, fgemm.strassen_plan(d, v))
    for key, e in figs.items():
        assert 1e-4 < e < 5e-3, key
    for dt in (BF, HF):
        for v in (fgemm.FGEMM_VARIANT_S69, fgemm.FGEMM_VARIANT_WINOGRAD):
            assert figs[dt, v, 2] > figs[dt, v, 1]                   # a level adds error
        for d in (1, 2):                                             # Winograd's chained sums
            assert figs[dt, fgemm.FGEMM_VARIANT_WINOGRAD, d] > figs[dt, fgemm.FGEMM_VARIANT_S69, d]
    assert fgemm.fgemm_plan_rel_err(7, cl) < 0
    assert fgemm.fgemm_plan_rel_err(BF, fgemm.strassen_plan(3, 0)) < 0


def test_select_crossover_with_calibrated_constants():
    """The decision at the sizes where Strassen starts to win on MI355X, under the
    constants a handle gets on that chip (eta_mfma 0.52, eta_hbm 0.66, workspace cap a
    third of 288 GB): classical at and below 40960^3 for bf16 inputs, at 32768^3 for
    fp16 ones (which run the classical kernel at a lower clock), two-level S69 from
    49152^3 on; a 16 GiB cap keeps classical (the plans need 42 and 75 GB)."""
    md = mi355x_model(eta_mfma=0.52, eta_hbm=0.66, max_workspace_bytes=288e9 / 3)
    path = lambda n, dt, m=md: (lambda p: (p.path, p.depth, p.variant))(select(n, n, n, m, dtype=dt))
    CL, S = fgemm.FGEMM_PATH_CLASSICAL, fgemm.FGEMM_PATH_STRASSEN
    S69 = fgemm.FGEMM_VARIANT_S69
    for n in (16384, 24576, 32768, 40960):
        assert path(n, BF)[0] == CL, n
    for n in (16384, 32768):
        assert path(n, HF)[0] == CL, n
    assert path(40960, HF) == (S, 1, S69)
    for n in (49152, 65536):
        for dt in (BF, HF):
            assert path(n, dt) == (S, 2, S69), (n, dt)
            p = select(n, n, n, md, dtype=dt)
            assert p.workspace_bytes <= md.max_workspace_bytes
            assert p.t_pred_us < p.t_classical_pred_us
    small_cap = mi355x_model(eta_mfma=0.52, eta_hbm=0.66)
    assert path(65536, BF, small_cap)[0] == CL


def test_split_k_respects_the_workspace_cap():
    """Split K needs slices*M*N*4 bytes of fp32 partials: a skinny shape that splits
    under the default cap stays unsplit when the cap is below the smallest split's
    need, and splits less when the cap admits only two slices."""
    md = mi355x_model(eta_mfma=0.52, eta_hbm=0.66)
    M, N, K = 64, 1024, 16384
    p = select(M, N, K, md)
    assert p.split_k > 2 and p.workspace_bytes == p.split_k * M * N * 4
    tight = mi355x_model(eta_mfma=0.52, eta_hbm=0.66, max_workspace_bytes=2 * M * N * 4 - 1)
    assert select(M, N, K, tight).split_k == 1
    two = mi355x_model(eta_mfma=0.52, eta_hbm=0.66, max_workspace_bytes=2 * M * N * 4)
    q = select(M, N, K, two)
    assert q.split_k == 2 and q.workspace_bytes <= two.max_workspace_bytes


def test_rectangular_scheme_error_figures_and_model_time():
    """The <2,2,3;11> scheme has an error figure at depth 1 only (below S69's at
    depth 1: two thirds of C are S69's, one third plain blocks), and the model never
    prefers it where Strassen's 2 x 2 split applies as well (eleven products of a
    twelfth of the work against seven of an eighth)."""
    r1 = fgemm.strassen_plan(1, fgemm.FGEMM_VARIANT_R223)
    r2 = fgemm.strassen_plan(2, fgemm.FGEMM_VARIANT_R223)
    s1 = fgemm.strassen_plan(1, fgemm.FGEMM_VARIANT_S69)
    for dt in (fgemm.FGEMM_BF16, fgemm.FGEMM_F16):
        assert 0 < fgemm.fgemm_plan_rel_err(dt, r1) < fgemm.fgemm_plan_rel_err(dt, s1)
        assert fgemm.fgemm_plan_rel_err(dt, r2) < 0
    m = mi355x_model()
    for (M, N, K) in [(16384, 24576, 16384), (49152, 49152, 49152), (32768, 49152, 32768)]:
        p = fgemm.fgemm_select_model(m, 0, 0, M, N, K, fgemm.FGEMM_BF16)
        assert p.variant != fgemm.FGEMM_VARIANT_R223 or p.path == fgemm.FGEMM_PATH_CLASSICAL


def test_read_probe_argument_checks():
    """Every refusal of fgemm_read_probe returns before any device call."""
    inval = fgemm.FGEMM_ERR_INVALID_VALUE
    fake = 1 << 20  # a 16-byte aligned address that is never dereferenced
    for src, nbytes, out in ((fake, -16, fake), (fake, 15, fake), (fake, 24, fake),
                             (fake, 32, None), (None, 16, fake), (fake + 8, 16, fake)):
        assert fgemm.fgemm_read_probe(src, nbytes, out, None, check=False) == inval


def test_quantize_argument_checks():
    """fgemm_quantize_mx's refusals return before any device call."""
    inval, nsup = fgemm.FGEMM_ERR_INVALID_VALUE, fgemm.FGEMM_ERR_NOT_SUPPORTED
    p = 1 << 20  # 16-byte aligned addresses that are never dereferenced

    def call(rows=64, cols=64, ldx=64, dt=fgemm.FGEMM_BF16, tr=0, fmt=fgemm.FGEMM_E4M3, x=p,
             q=p, ldq=64, s=p, lds=2):
        return fgemm.fgemm_quantize_mx(x, rows, cols, ldx, dt, tr, fmt, q, ldq, s, lds, None,
                                       check=False)
    assert call(cols=48) == inval                    # row length not a multiple of 32
    assert call(tr=1, rows=40) == inval              # transposed row length = rows
    assert call(ldx=32) == inval                     # ldx < cols
    assert call(ldq=63) == inval                     # a quantized row is 64 bytes
    assert call(fmt=fgemm.FGEMM_E2M1, ldq=31) == inval   # 4-bit: 32 bytes
    assert call(lds=1) == inval
    assert call(fmt=5) == inval and call(dt=3) == inval
    assert call(x=0) == inval and call(q=0) == inval and call(s=0) == inval
    assert call(x=p + 4) == nsup and call(q=p + 8) == nsup
    assert call(ldx=68) == nsup and call(ldq=72) == nsup
    assert call(rows=0, x=0, q=0, s=0) == fgemm.FGEMM_OK   # nothing to do
