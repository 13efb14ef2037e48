// host_harness.cpp — drives the host-only entry points of the C ABI (argument
// checks, the decision model, the quantization helpers, the error model, status
// strings, handle-less refusals) over a grid of shapes, layouts, types, epilogues
// and model constants, built with AddressSanitizer and UndefinedBehaviorSanitizer.
// It checks a few properties on the way and prints one summary line; any
// sanitizer report fails the run.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fgemm.h"

static int failures = 0;
#define EXPECT(c)                                                  \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "harness: %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static fgemm_model_t model(double hbm, double eta, double ws, double err) {
  fgemm_model_t m;
  memset(&m, 0, sizeof(m));
  m.compute_units = 256;
  m.peak_tflops = 256 * 4096.0 * 2.4e9 / 1e12;
  m.hbm_gbps = hbm;
  m.eta_mfma = eta;
  m.eta_hbm = 0.66;
  m.launch_us = 4.0;
  m.max_workspace_bytes = ws;
  m.max_rel_err = err;
  return m;
}

int main() {
  static const int64_t dims[] = {0, 1, 7, 8, 63, 64, 65, 255, 256, 257, 1000, 4096, 8192,
                                 14336, 16384, 40960, 49152, 65536, 1 << 20};
  const int nd = (int)(sizeof(dims) / sizeof(dims[0]));
  static const uint32_t flag_sets[] = {0u,
                                       FGEMM_EPI_BIAS,
                                       FGEMM_EPI_ROWSUMSQ,
                                       FGEMM_EPI_BIAS | FGEMM_EPI_ROWSUMSQ,
                                       FGEMM_EPI_RMS_SWIGLU,
                                       FGEMM_EPI_ACT | FGEMM_EPI_BIAS,
                                       FGEMM_EPI_ROPE,
                                       FGEMM_EPI_SWIGLU_BWD,
                                       FGEMM_EPI_RMS_BWD};
  const fgemm_model_t models[] = {model(8000, 0.52, 96e9, 5e-3), model(80000, 0.7, 16e9, 5e-3),
                                  model(800, 0.7, 1e6, 1e-3), model(8000, 0.52, 1e18, 5e-4)};
  void* const P = (void*)(uintptr_t)0x10000;  // never dereferenced
  long selects = 0, checks = 0;
  double tsum = 0;
  for (int mi = 0; mi < 4; ++mi)
    for (int a = 0; a < nd; ++a)
      for (int b = 0; b < nd; ++b)
        for (int c = 0; c < nd; c += 2)
          for (int f = 0; f < 9; ++f)
            for (int dt = 0; dt < 2; ++dt) {
              const int64_t M = dims[a], N = dims[b], K = dims[c];
              fgemm_epilogue_t e;
              memset(&e, 0, sizeof(e));
              e.flags = flag_sets[f];
              e.bias = P; e.rowsumsq = (float*)P; e.rms_rowsumsq = (const float*)P;
              e.rms_n = 4096; e.rms_eps = 1e-6f; e.act = FGEMM_ACT_GELU_TANH;
              e.rope_head_dim = 64; e.rope_theta = 10000.f;
              e.swiglu_dout = P; e.swiglu_ldd = N > 0 ? N : 1;
              e.rms_grad = (float*)P; e.rms_x = P; e.rms_ldx = N > 0 ? N : 1;
              fgemm_plan_t p;
              fgemm_status_t s = fgemm_select_model(&models[mi], (fgemm_op_t)(f & 1),
                                                    (fgemm_op_t)((a + b) & 1), M, N, K,
                                                    (fgemm_dtype_t)dt, &e, &p);
              ++selects;
              if (s == FGEMM_OK) {
                EXPECT(p.t_pred_us >= 0 && isfinite(p.t_pred_us));
                EXPECT(p.t_pred_us <= p.t_classical_pred_us + 1e-9);
                EXPECT(p.pred_rel_err > 0 && p.pred_rel_err <= models[mi].max_rel_err + 1e-12);
                if (p.path == FGEMM_PATH_STRASSEN) {
                  EXPECT(M % 16 == 0 && K % 16 == 0);
                  EXPECT(!(e.flags & FGEMM_EPI_ROWSUMSQ));  // the statistics guard
                  EXPECT(p.workspace_bytes <= models[mi].max_workspace_bytes);
                }
                tsum += p.t_pred_us * 1e-9;
              }
              const int64_t Nb = (e.flags & (FGEMM_EPI_RMS_SWIGLU | FGEMM_EPI_SWIGLU_BWD)) ? 2 * N : N;
              const int64_t Nc = (e.flags & FGEMM_EPI_SWIGLU_BWD) ? 2 * N : N;
              for (int ta = 0; ta < 2; ++ta) {
                const int64_t lda = ta ? (M > 0 ? M : 1) : (K > 0 ? K : 1);
                const int64_t ldb = (K > 0 ? K : 1) > Nb ? (K > 0 ? K : 1) : (Nb > 0 ? Nb : 1);
                fgemm_status_t st = fgemm_check_args((fgemm_op_t)ta, FGEMM_OP_T, M, N, K, P, lda,
                                                     P, ldb, 0.f, P, Nc > 0 ? Nc : 1,
                                                     (fgemm_dtype_t)dt, &e);
                ++checks;
                EXPECT(st == FGEMM_OK || st == FGEMM_ERR_NOT_SUPPORTED ||
                       st == FGEMM_ERR_INVALID_VALUE);
                // a too-small leading dimension is always refused
                if (M > 1 && K > 1)
                  EXPECT(fgemm_check_args((fgemm_op_t)ta, FGEMM_OP_T, M, N, K, P, lda - 1, P, ldb,
                                          0.f, P, Nc > 0 ? Nc : 1, (fgemm_dtype_t)dt, &e) ==
                         FGEMM_ERR_INVALID_VALUE);
                ++checks;
              }
            }
  // quantization helpers and the error model
  for (int a = 0; a < nd; ++a)
    for (int b = 0; b < nd; ++b) {
      const int64_t t = fgemm_tile_count(dims[a], dims[b], 256, 128);
      EXPECT(t >= 0);
      double tail = -1;
      const int64_t w = fgemm_wave_count(t, 256, &tail);
      EXPECT(w >= 0 && tail >= 0 && tail <= 1);
    }
  EXPECT(fgemm_tile_count(-1, 1, 1, 1) == -1 && fgemm_wave_count(1, 0, NULL) == -1);
  for (int dt = -1; dt < 3; ++dt)
    for (int path = -1; path < 3; ++path)
      for (int d = -1; d < 4; ++d)
        for (int v = -1; v < 3; ++v) {
          fgemm_plan_t p;
          memset(&p, 0, sizeof(p));
          p.path = path; p.depth = d; p.variant = v;
          const double r = fgemm_plan_rel_err((fgemm_dtype_t)dt, &p);
          EXPECT(r < 0 || (r > 0 && r < 1e-2));
        }
  EXPECT(fgemm_plan_rel_err(FGEMM_BF16, NULL) < 0);
  for (int s = -2; s < 8; ++s) EXPECT(fgemm_status_string((fgemm_status_t)s) != NULL);
  // handle-less and malformed calls are refused without touching anything
  fgemm_plan_t p;
  EXPECT(fgemm_select(NULL, FGEMM_OP_N, FGEMM_OP_N, 8, 8, 8, FGEMM_BF16, NULL, &p) ==
         FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_gemm(NULL, FGEMM_OP_N, FGEMM_OP_N, 8, 8, 8, 1.f, P, 8, P, 8, 0.f, P, 8, FGEMM_BF16,
                    NULL, NULL) == FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_gemm_noalloc(NULL, FGEMM_OP_N, FGEMM_OP_N, 8, 8, 8, 1.f, P, 8, P, 8, 0.f, P, 8,
                            FGEMM_BF16, NULL, NULL) == FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_select_model(NULL, FGEMM_OP_N, FGEMM_OP_N, 8, 8, 8, FGEMM_BF16, NULL, &p) ==
         FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_gemm_f8(NULL, 8, 8, 128, 1.f, P, 128, FGEMM_E4M3, 1.f, P, 128, FGEMM_E4M3, 1.f, 0.f,
                       P, 8, FGEMM_BF16, NULL, NULL) == FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_gemm_mxf8(NULL, 8, 8, 128, 1.f, P, 128, FGEMM_E4M3, P, 16, P, 128, FGEMM_E4M3, P, 16,
                         0.f, P, 8, FGEMM_BF16, NULL, NULL) == FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_create(NULL, 0) == FGEMM_ERR_INVALID_VALUE);
  EXPECT(fgemm_destroy(NULL) == FGEMM_ERR_INVALID_VALUE);
  printf("harness: %ld selects, %ld checks, sum %.6f, %d failures\n", selects, checks, tsum,
         failures);
  return failures ? 1 : 0;
}
