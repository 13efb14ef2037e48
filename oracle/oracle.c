/*
 * oracle.c — plain, slow, obviously-correct CPU reference for the half-precision
 * GEMM path.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the smoke
 * check and by the CPU-baseline leg of the benchmark, never by the product path.
 * It shares no code, header, table or constant with the GPU library.
 *
 * What it computes (all in IEEE fp64, from the exact 16-bit input values):
 *
 *   D = alpha * op(A) * op(B) + beta * C_in  [+ bias_j]          (HGEMM, fp32+ acc)
 *   out = Q(D)            Q = round-to-nearest-even to the output 16-bit type
 *
 *   Sources:
 *   - "CUDA-L2: Surpassing cuBLAS Performance for Matrix Multiplication through
 *     Reinforcement Learning" (chatpaper.ai), abstract: the operation is HGEMM,
 *     half-precision general matrix multiply, in NN and TN layouts.
 *   - CS336 Lecture 05 notes (jw9603.github.io), Page 26 "Low precision drives
 *     faster matrix multiplies": 16-bit products accumulated in a wider type.
 *   - tilnote.io PingPong GEMM note, opening section: a GEMM is a mainloop plus an
 *     epilogue that scales and applies elementwise operations before the store.
 *   - same note, section on CODA: the first GEMM's epilogue produces per-row norm
 *     statistics, the second GEMM's epilogue applies the norm scaling, and SwiGLU
 *     is fused into an epilogue.
 *   - FalconGEMM (euno.news summary), Methodology items 1 and 4: Strassen-like and
 *     Winograd-based low-complexity algorithms with a recursion depth; the
 *     recursion reaches the same product with fewer multiplications.
 *
 * Accumulation: each element's k-sum runs in ascending k in fp64 (rows and
 * columns may be blocked, k-order never changes, so the result is bitwise that of
 * the naive triple loop).  Products of two 16-bit values are exact in fp64.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - epilogue order: D = alpha*acc + beta*C_in + bias, then Q, then statistics;
 *   - the sum of squares is taken over the rounded (written) output row;
 *   - RMS_SWIGLU: r_i = 1/sqrt(ss_i/n + eps); g = r_i*alpha*H[i][j],
 *     u = r_i*alpha*H[i][j+Nout]; out = Q(silu(g)*u + beta*C_in[i][j]);
 *     silu(x) = x/(1+exp(-x)); B then has 2*Nout columns (gate block, up block).
 *   - ACT and ROPE (the same note's opening and CODA sections: elementwise work and
 *     RoPE run in the epilogue) transform the full linear result before rounding:
 *     out = Q(T(alpha*acc + beta*C_in + bias)).
 *     ACT: relu(x) = max(x, 0); silu as above; gelu = the tanh approximation of
 *     Hendrycks and Gimpel, 0.5*x*(1 + tanh(sqrt(2/pi)*(x + 0.044715*x^3))).
 *     ROPE: rotary position embedding of Su et al. (RoFormer) on interleaved pairs:
 *     column j lies in head j / hd at offset d = j % hd, pair p = d / 2 rotates by
 *     theta_ij = pos_i * base^(-2p/hd):
 *       y[2p] = x[2p] cos(theta) - x[2p+1] sin(theta)
 *       y[2p+1] = x[2p] sin(theta) + x[2p+1] cos(theta).
 *   - SWIGLU_BWD, the backward of RMS_SWIGLU with the row scale r_i held fixed (the
 *     same note's CODA section: backward passes of SwiGLU can run in the epilogue):
 *     recompute H = op(A)op(B) (gate | up, 2*Nout columns) and, with g, u as in the
 *     forward and dO the incoming gradient, write the gradient with respect to H:
 *       out[i][j]        = Q(dO[i][j] * u * silu'(g) * r_i * alpha)
 *       out[i][Nout + j] = Q(dO[i][j] * silu(g) * r_i * alpha)
 *     silu'(x) = s(x)(1 + x(1 - s(x))), s(x) = 1/(1+exp(-x)).  It also gives the
 *     gradient with respect to the row scale, rgrad_i = sum_j dO (silu'(g) g u +
 *     silu(g) u) / r_i.
 *   - RMS_BWD, the rest of the RMSNorm backward (r_i = 1/sqrt(ss_i/n + eps),
 *     ss_i = sum_k X_ik^2, so dr_i/dX_ik = -r_i^3 X_ik / n): a GEMM's epilogue adds
 *     the scale's contribution to the gradient of X,
 *       out = Q(alpha*acc + c_i * X_ij),  c_i = -r_i^3 * rgrad_i / n.
 *   - Strassen recursion keeps fp64 temporaries (it is the exact identity check).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F16 0
#define OR_BF16 1

#define OR_EPI_BIAS 1
#define OR_EPI_ROWSUMSQ 2
#define OR_EPI_RMS_SWIGLU 4
#define OR_EPI_ACT 8
#define OR_EPI_ROPE 16

#define OR_ACT_RELU 1
#define OR_ACT_SILU 2
#define OR_ACT_GELU_TANH 3

/* ---------------------------------------------------------------------------
 * 16-bit decode: exact value of an IEEE binary16 or bfloat16 bit pattern.
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 * ------------------------------------------------------------------------- */
double oracle_decode(uint16_t h, int dtype) {
    int sign = (h >> 15) & 1;
    int ebits = dtype == OR_F16 ? 5 : 8;
    int fbits = dtype == OR_F16 ? 10 : 7;
    int bias = dtype == OR_F16 ? 15 : 127;
    int emax = (1 << ebits) - 1;
    int e = (h >> fbits) & emax;
    int f = h & ((1 << fbits) - 1);
    double v;
    if (e == emax) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, 1 - bias - fbits); /* subnormal: f * 2^(1-bias-fbits) */
    } else {
        v = ldexp((double)((1 << fbits) | f), e - bias - fbits);
    }
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------------
 * 16-bit encode with round-to-nearest, ties to even, straight from fp64.
 * The quantum (ulp) of the target format at |x| is a power of two; x/ulp is
 * exact, rint() in the default rounding mode rounds half to even, and the
 * product by ulp is exact again.  Overflow of the rounded value gives inf.
 * ------------------------------------------------------------------------- */
uint16_t oracle_encode(double x, int dtype) {
    int fbits = dtype == OR_F16 ? 10 : 7;
    int bias = dtype == OR_F16 ? 15 : 127;
    int ebits = dtype == OR_F16 ? 5 : 8;
    int emax_field = (1 << ebits) - 1;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(emax_field << fbits | (1 << (fbits - 1)));
    double a = fabs(x);
    int emin = 1 - bias;                 /* exponent of the smallest normal */
    int emax = bias;                     /* exponent of the largest finite  */
    double maxval = ldexp(2.0 - ldexp(1.0, -fbits), emax);
    if (isinf(a)) return sign | (uint16_t)(emax_field << fbits);
    int e2;
    frexp(a, &e2);                       /* a = m * 2^e2, 0.5 <= m < 1 */
    int ex = e2 - 1;                     /* a in [2^ex, 2^(ex+1)) */
    if (a == 0.0) return sign;
    if (ex < emin) ex = emin;            /* subnormal range shares emin's quantum */
    double ulp = ldexp(1.0, ex - fbits);
    double r = rint(a / ulp) * ulp;
    if (r > maxval) return sign | (uint16_t)(emax_field << fbits);
    if (r == 0.0) return sign;
    /* pack the exact value r */
    frexp(r, &e2);
    ex = e2 - 1;
    if (ex < emin) { /* subnormal */
        uint16_t f = (uint16_t)(r / ldexp(1.0, emin - fbits));
        return sign | f;
    }
    double mant = r / ldexp(1.0, ex) - 1.0;            /* in [0,1) */
    uint16_t f = (uint16_t)(mant * (double)(1 << fbits));
    uint16_t e = (uint16_t)(ex + bias);
    return sign | (uint16_t)(e << fbits) | f;
}

void oracle_decode_array(const uint16_t* h, double* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode(h[i], dtype);
}

void oracle_encode_array(const double* x, uint16_t* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode(x[i], dtype);
}

/* ---------------------------------------------------------------------------
 * Classical GEMM rows.
 * op(A)[i][k] = transA ? A[k*lda + i] : A[i*lda + k]   (row-major storage)
 * op(B)[k][j] = transB ? B[j*ldb + k] : B[k*ldb + j]
 * The selected rows `rows[0..nrows)` of D (nrows x Ncols, Ncols = N) are computed.
 * ------------------------------------------------------------------------- */
typedef struct {
    int transA, transB;
    int64_t M, N, K;
    const uint16_t* A; int64_t lda;
    const uint16_t* B; int64_t ldb;
    int dtype;
    const double* Bd;     /* decoded op(B), K x N row-major */
    const int64_t* rows; int64_t nrows;
    double* H;            /* nrows x N: the raw k-sums */
    int64_t r0, r1;       /* this worker's slice of `rows` */
} gemm_job_t;

#define OR_JB 512

static void* gemm_worker(void* p) {
    gemm_job_t* J = (gemm_job_t*)p;
    int64_t K = J->K, N = J->N;
    double* arow = (double*)malloc(sizeof(double) * (K > 0 ? K : 1));
    for (int64_t r = J->r0; r < J->r1; ++r) {
        int64_t i = J->rows[r];
        for (int64_t k = 0; k < K; ++k) {
            uint16_t h = J->transA ? J->A[k * J->lda + i] : J->A[i * J->lda + k];
            arow[k] = oracle_decode(h, J->dtype);
        }
        double* hrow = J->H + r * N;
        for (int64_t j = 0; j < N; ++j) hrow[j] = 0.0;
        /* ascending k for every element of the row: hrow[j] = sum_k a_k * b_kj */
        for (int64_t jb = 0; jb < N; jb += OR_JB) {
            int64_t je = jb + OR_JB < N ? jb + OR_JB : N;
            for (int64_t k = 0; k < K; ++k) {
                double a = arow[k];
                const double* brow = J->Bd + k * N;
                for (int64_t j = jb; j < je; ++j) hrow[j] += a * brow[j];
            }
        }
    }
    free(arow);
    return NULL;
}

static void decode_opB(int transB, int64_t K, int64_t N, const uint16_t* B, int64_t ldb,
                       int dtype, double* Bd) {
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            uint16_t h = transB ? B[j * ldb + k] : B[k * ldb + j];
            Bd[k * N + j] = oracle_decode(h, dtype);
        }
}

/* H[r][j] = sum_k op(A)[rows[r]][k] * op(B)[k][j], fp64, ascending k. */
static int raw_products(int transA, int transB, int64_t M, int64_t N, int64_t K,
                        const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        int dtype, const int64_t* rows, int64_t nrows, double* H,
                        int nthreads) {
    (void)M;
    double* Bd = (double*)malloc(sizeof(double) * (K * N > 0 ? K * N : 1));
    if (!Bd) return -1;
    decode_opB(transB, K, N, B, ldb, dtype, Bd);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    gemm_job_t jobs[256];
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int launched = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = t * per, r1 = r0 + per < nrows ? r0 + per : nrows;
        if (r0 >= r1) break;
        gemm_job_t j = {transA, transB, M, N, K, A, lda, B, ldb, dtype, Bd, rows, nrows, H, r0, r1};
        jobs[t] = j;
        pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
        ++launched;
    }
    for (int t = 0; t < launched; ++t) pthread_join(th[t], NULL);
    free(Bd);
    return 0;
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

static double activation(int act, double x) {
    const double pi = 3.14159265358979323846;
    switch (act) {
        case OR_ACT_RELU: return x > 0.0 ? x : 0.0;
        case OR_ACT_SILU: return silu(x);
        case OR_ACT_GELU_TANH: return 0.5 * x * (1.0 + tanh(sqrt(2.0 / pi) * (x + 0.044715 * x * x * x)));
    }
    return x;
}

/*
 * oracle_gemm: classical reference with the epilogues.
 *   N is the width of op(B) (for RMS_SWIGLU, N = 2*Nout and the output is Nout wide).
 *   C_in, when beta != 0, is Mout x Nout with leading dimension ldc.
 *   Outputs for the selected rows: D (nrows x Nout, unrounded fp64),
 *   Q (nrows x Nout, 16-bit RNE bits), ss (nrows, only for ROWSUMSQ).
 * Returns 0 on success, -1 on bad arguments.
 */
int oracle_gemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                   const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, double beta,
                   const uint16_t* Cin, int64_t ldc, int dtype, int epi, const uint16_t* bias,
                   const double* rms_ss, int64_t rms_n, double rms_eps, int act,
                   const int64_t* rope_pos, int64_t rope_hd, double rope_base,
                   const int64_t* rows, int64_t nrows, double* D, uint16_t* Q, double* ss,
                   int nthreads) {
    int swiglu = (epi & OR_EPI_RMS_SWIGLU) != 0;
    int rope = (epi & OR_EPI_ROPE) != 0;
    if (swiglu && (epi & (OR_EPI_BIAS | OR_EPI_ROWSUMSQ | OR_EPI_ACT | OR_EPI_ROPE))) return -1;
    if ((epi & OR_EPI_ACT) && rope) return -1;
    if ((epi & OR_EPI_ACT) && (act < OR_ACT_RELU || act > OR_ACT_GELU_TANH)) return -1;
    if (rope && (rope_hd <= 0 || rope_hd % 2 || N % rope_hd || !rope_pos || !(rope_base > 0.0)))
        return -1;
    if (swiglu && (N % 2)) return -1;
    int64_t Nout = swiglu ? N / 2 : N;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    double* H = (double*)malloc(sizeof(double) * (nrows * N > 0 ? nrows * N : 1));
    if (!H) return -1;
    if (raw_products(transA, transB, M, N, K, A, lda, B, ldb, dtype, rows, nrows, H, nthreads)) {
        free(H);
        return -1;
    }
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        const double* h = H + r * N;
        double sum_sq = 0.0;
        double rscale = 1.0;
        if (swiglu) rscale = 1.0 / sqrt(rms_ss[r] / (double)rms_n + rms_eps);
        for (int64_t j = 0; j < Nout; ++j) {
            double d;
            if (swiglu) {
                double g = rscale * (alpha * h[j]);
                double u = rscale * (alpha * h[j + Nout]);
                d = silu(g) * u;
            } else {
                d = alpha * h[j];
            }
            if (beta != 0.0) d += beta * oracle_decode(Cin[i * ldc + j], dtype);
            if (epi & OR_EPI_BIAS) d += oracle_decode(bias[j], dtype);
            if (epi & OR_EPI_ACT) d = activation(act, d);
            D[r * Nout + j] = d;
        }
        if (rope) {
            /* rotate each interleaved pair of the row's linear results */
            for (int64_t j = 0; j < Nout; j += 2) {
                int64_t p = (j % rope_hd) / 2;
                double theta = (double)rope_pos[r] * pow(rope_base, -2.0 * (double)p / (double)rope_hd);
                double x0 = D[r * Nout + j], x1 = D[r * Nout + j + 1];
                D[r * Nout + j] = x0 * cos(theta) - x1 * sin(theta);
                D[r * Nout + j + 1] = x0 * sin(theta) + x1 * cos(theta);
            }
        }
        for (int64_t j = 0; j < Nout; ++j) {
            uint16_t q = oracle_encode(D[r * Nout + j], dtype);
            Q[r * Nout + j] = q;
            if (epi & OR_EPI_ROWSUMSQ) {
                double qv = oracle_decode(q, dtype);
                sum_sq += qv * qv;
            }
        }
        if ((epi & OR_EPI_ROWSUMSQ) && ss) ss[r] = sum_sq;
    }
    free(H);
    return 0;
}

/*
 * oracle_swiglu_bwd: N is the width of op(B) (2*Nout).  dO holds the incoming
 * gradient of the selected rows (nrows x Nout, fp64), rms_ss their sums of squares.
 * Outputs D (nrows x N, unrounded) and Q (nrows x N, 16-bit RNE bits).
 */
int oracle_swiglu_bwd(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                      const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int dtype,
                      const double* dO, const double* rms_ss, int64_t rms_n, double rms_eps,
                      const int64_t* rows, int64_t nrows, double* D, uint16_t* Q, double* rgrad,
                      int nthreads) {
    if (N % 2 || rms_n <= 0) return -1;
    int64_t Nout = N / 2;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    double* H = (double*)malloc(sizeof(double) * (nrows * N > 0 ? nrows * N : 1));
    if (!H) return -1;
    if (raw_products(transA, transB, M, N, K, A, lda, B, ldb, dtype, rows, nrows, H, nthreads)) {
        free(H);
        return -1;
    }
    for (int64_t r = 0; r < nrows; ++r) {
        const double* h = H + r * N;
        double rr = 1.0 / sqrt(rms_ss[r] / (double)rms_n + rms_eps);
        double rs = alpha * rr;
        double acc_r = 0.0;
        for (int64_t j = 0; j < Nout; ++j) {
            double g = rs * h[j], u = rs * h[j + Nout];
            double s = 1.0 / (1.0 + exp(-g));
            double d = dO[r * Nout + j];
            double dg = d * u * s * (1.0 + g * (1.0 - s)) * rs;
            double du = d * g * s * rs;
            acc_r += d * (s * (1.0 + g * (1.0 - s)) * g * u + g * s * u);
            D[r * N + j] = dg;
            D[r * N + Nout + j] = du;
            Q[r * N + j] = oracle_encode(dg, dtype);
            Q[r * N + Nout + j] = oracle_encode(du, dtype);
        }
        if (rgrad) rgrad[r] = acc_r / rr;
    }
    free(H);
    return 0;
}

/*
 * oracle_rms_bwd: out = Q(alpha*op(A)op(B) + c_i * X_ij), c_i = -r_i^3 * rgrad_i / n,
 * r_i = 1/sqrt(ss_i/n + eps).  X (the normalised layer's input, decoded, selected
 * rows, nrows x N), rms_ss and rgrad are per selected row.
 */
int oracle_rms_bwd(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                   const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int dtype,
                   const double* X, const double* rms_ss, const double* rgrad, int64_t rms_n,
                   double rms_eps, const int64_t* rows, int64_t nrows, double* D, uint16_t* Q,
                   int nthreads) {
    if (rms_n <= 0) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    double* H = (double*)malloc(sizeof(double) * (nrows * N > 0 ? nrows * N : 1));
    if (!H) return -1;
    if (raw_products(transA, transB, M, N, K, A, lda, B, ldb, dtype, rows, nrows, H, nthreads)) {
        free(H);
        return -1;
    }
    for (int64_t r = 0; r < nrows; ++r) {
        double rr = 1.0 / sqrt(rms_ss[r] / (double)rms_n + rms_eps);
        double c = -rr * rr * rr * rgrad[r] / (double)rms_n;
        for (int64_t j = 0; j < N; ++j) {
            double d = alpha * H[r * N + j] + c * X[r * N + j];
            D[r * N + j] = d;
            Q[r * N + j] = oracle_encode(d, dtype);
        }
    }
    free(H);
    return 0;
}

int oracle_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, double beta,
                const uint16_t* Cin, int64_t ldc, int dtype, int epi, const uint16_t* bias,
                const double* rms_ss, int64_t rms_n, double rms_eps, const int64_t* rows,
                int64_t nrows, double* D, uint16_t* Q, double* ss, int nthreads) {
    if (epi & (OR_EPI_ACT | OR_EPI_ROPE)) return -1;
    return oracle_gemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, Cin, ldc, dtype,
                          epi, bias, rms_ss, rms_n, rms_eps, 0, NULL, 0, 0.0, rows, nrows, D, Q,
                          ss, nthreads);
}

/* ---------------------------------------------------------------------------
 * Strassen / Winograd recursion in fp64 (identity check and diagnostic).
 * Matrices here are dense row-major double blocks with their own stride.
 * variant 0: Strassen (1969), seven products M1..M7 and 18 block additions.
 * variant 1: Winograd's form, seven products P1..P7 and 15 block additions.
 * depth 0 falls back to the classical loop (ascending k).
 * ------------------------------------------------------------------------- */
typedef struct { double* p; int64_t r, c, ld; } blk_t;

static blk_t blk_alloc(int64_t r, int64_t c) {
    blk_t b = {(double*)calloc((size_t)(r * c > 0 ? r * c : 1), sizeof(double)), r, c, c};
    return b;
}
static blk_t blk_sub(blk_t m, int bi, int bj) {
    blk_t b = {m.p + bi * (m.r / 2) * m.ld + bj * (m.c / 2), m.r / 2, m.c / 2, m.ld};
    return b;
}
#define AT(b, i, j) ((b).p[(i) * (b).ld + (j)])

/* out = x + sy*y  (sy = +1 or -1), elementwise */
static void blk_axpy(blk_t out, blk_t x, blk_t y, double sy) {
    for (int64_t i = 0; i < out.r; ++i)
        for (int64_t j = 0; j < out.c; ++j) AT(out, i, j) = AT(x, i, j) + sy * AT(y, i, j);
}
static void blk_copy(blk_t out, blk_t x) {
    for (int64_t i = 0; i < out.r; ++i)
        for (int64_t j = 0; j < out.c; ++j) AT(out, i, j) = AT(x, i, j);
}

static void classical(blk_t C, blk_t A, blk_t B) {
    for (int64_t i = 0; i < C.r; ++i) {
        for (int64_t j = 0; j < C.c; ++j) AT(C, i, j) = 0.0;
        for (int64_t k = 0; k < A.c; ++k) {
            double a = AT(A, i, k);
            for (int64_t j = 0; j < C.c; ++j) AT(C, i, j) += a * AT(B, k, j);
        }
    }
}

static void strassen_rec(blk_t C, blk_t A, blk_t B, int depth, int variant);

static void s69(blk_t C, blk_t A, blk_t B, int depth) {
    int64_t m = A.r / 2, k = A.c / 2, n = B.c / 2;
    blk_t A11 = blk_sub(A, 0, 0), A12 = blk_sub(A, 0, 1), A21 = blk_sub(A, 1, 0), A22 = blk_sub(A, 1, 1);
    blk_t B11 = blk_sub(B, 0, 0), B12 = blk_sub(B, 0, 1), B21 = blk_sub(B, 1, 0), B22 = blk_sub(B, 1, 1);
    blk_t C11 = blk_sub(C, 0, 0), C12 = blk_sub(C, 0, 1), C21 = blk_sub(C, 1, 0), C22 = blk_sub(C, 1, 1);
    blk_t L = blk_alloc(m, k), R = blk_alloc(k, n);
    blk_t Mx[7];
    for (int t = 0; t < 7; ++t) Mx[t] = blk_alloc(m, n);
    /* M1 = (A11 + A22)(B11 + B22) */
    blk_axpy(L, A11, A22, 1); blk_axpy(R, B11, B22, 1); strassen_rec(Mx[0], L, R, depth - 1, 0);
    /* M2 = (A21 + A22) B11 */
    blk_axpy(L, A21, A22, 1); strassen_rec(Mx[1], L, B11, depth - 1, 0);
    /* M3 = A11 (B12 - B22) */
    blk_axpy(R, B12, B22, -1); strassen_rec(Mx[2], A11, R, depth - 1, 0);
    /* M4 = A22 (B21 - B11) */
    blk_axpy(R, B21, B11, -1); strassen_rec(Mx[3], A22, R, depth - 1, 0);
    /* M5 = (A11 + A12) B22 */
    blk_axpy(L, A11, A12, 1); strassen_rec(Mx[4], L, B22, depth - 1, 0);
    /* M6 = (A21 - A11)(B11 + B12) */
    blk_axpy(L, A21, A11, -1); blk_axpy(R, B11, B12, 1); strassen_rec(Mx[5], L, R, depth - 1, 0);
    /* M7 = (A12 - A22)(B21 + B22) */
    blk_axpy(L, A12, A22, -1); blk_axpy(R, B21, B22, 1); strassen_rec(Mx[6], L, R, depth - 1, 0);
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double m1 = AT(Mx[0], i, j), m2 = AT(Mx[1], i, j), m3 = AT(Mx[2], i, j);
            double m4 = AT(Mx[3], i, j), m5 = AT(Mx[4], i, j), m6 = AT(Mx[5], i, j);
            double m7 = AT(Mx[6], i, j);
            AT(C11, i, j) = m1 + m4 - m5 + m7;   /* C11 = M1 + M4 - M5 + M7 */
            AT(C12, i, j) = m3 + m5;             /* C12 = M3 + M5 */
            AT(C21, i, j) = m2 + m4;             /* C21 = M2 + M4 */
            AT(C22, i, j) = m1 - m2 + m3 + m6;   /* C22 = M1 - M2 + M3 + M6 */
        }
    free(L.p); free(R.p);
    for (int t = 0; t < 7; ++t) free(Mx[t].p);
}

static void winograd(blk_t C, blk_t A, blk_t B, int depth) {
    int64_t m = A.r / 2, k = A.c / 2, n = B.c / 2;
    blk_t A11 = blk_sub(A, 0, 0), A12 = blk_sub(A, 0, 1), A21 = blk_sub(A, 1, 0), A22 = blk_sub(A, 1, 1);
    blk_t B11 = blk_sub(B, 0, 0), B12 = blk_sub(B, 0, 1), B21 = blk_sub(B, 1, 0), B22 = blk_sub(B, 1, 1);
    blk_t C11 = blk_sub(C, 0, 0), C12 = blk_sub(C, 0, 1), C21 = blk_sub(C, 1, 0), C22 = blk_sub(C, 1, 1);
    blk_t S1 = blk_alloc(m, k), S2 = blk_alloc(m, k), S3 = blk_alloc(m, k), S4 = blk_alloc(m, k);
    blk_t T1 = blk_alloc(k, n), T2 = blk_alloc(k, n), T3 = blk_alloc(k, n), T4 = blk_alloc(k, n);
    blk_axpy(S1, A21, A22, 1);   /* S1 = A21 + A22 */
    blk_axpy(S2, S1, A11, -1);   /* S2 = S1 - A11  */
    blk_axpy(S3, A11, A21, -1);  /* S3 = A11 - A21 */
    blk_axpy(S4, A12, S2, -1);   /* S4 = A12 - S2  */
    blk_axpy(T1, B12, B11, -1);  /* T1 = B12 - B11 */
    blk_axpy(T2, B22, T1, -1);   /* T2 = B22 - T1  */
    blk_axpy(T3, B22, B12, -1);  /* T3 = B22 - B12 */
    blk_axpy(T4, T2, B21, -1);   /* T4 = T2 - B21  */
    blk_t P[7];
    for (int t = 0; t < 7; ++t) P[t] = blk_alloc(m, n);
    strassen_rec(P[0], A11, B11, depth - 1, 1); /* P1 = A11 B11 */
    strassen_rec(P[1], A12, B21, depth - 1, 1); /* P2 = A12 B21 */
    strassen_rec(P[2], S4, B22, depth - 1, 1);  /* P3 = S4 B22  */
    strassen_rec(P[3], A22, T4, depth - 1, 1);  /* P4 = A22 T4  */
    strassen_rec(P[4], S1, T1, depth - 1, 1);   /* P5 = S1 T1   */
    strassen_rec(P[5], S2, T2, depth - 1, 1);   /* P6 = S2 T2   */
    strassen_rec(P[6], S3, T3, depth - 1, 1);   /* P7 = S3 T3   */
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double p1 = AT(P[0], i, j), p2 = AT(P[1], i, j), p3 = AT(P[2], i, j);
            double p4 = AT(P[3], i, j), p5 = AT(P[4], i, j), p6 = AT(P[5], i, j);
            double p7 = AT(P[6], i, j);
            double u2 = p1 + p6;          /* U2 = P1 + P6 */
            double u3 = u2 + p7;          /* U3 = U2 + P7 */
            double u4 = u2 + p5;          /* U4 = U2 + P5 */
            AT(C11, i, j) = p1 + p2;      /* C11 = P1 + P2 */
            AT(C12, i, j) = u4 + p3;      /* C12 = U4 + P3 */
            AT(C21, i, j) = u3 - p4;      /* C21 = U3 - P4 */
            AT(C22, i, j) = u3 + p5;      /* C22 = U3 + P5 */
        }
    free(S1.p); free(S2.p); free(S3.p); free(S4.p);
    free(T1.p); free(T2.p); free(T3.p); free(T4.p);
    for (int t = 0; t < 7; ++t) free(P[t].p);
}

static void strassen_rec(blk_t C, blk_t A, blk_t B, int depth, int variant) {
    if (depth <= 0) {
        classical(C, A, B);
        return;
    }
    if (variant == 0) s69(C, A, B, depth);
    else winograd(C, A, B, depth);
}

/*
 * oracle_strassen: C = op(A)*op(B) (fp64, no epilogue) through `depth` levels of
 * the 2x2 block recursion.  M, N, K must be divisible by 2^depth.
 * The 16-bit inputs are decoded exactly; out is M x N fp64 row-major.
 */
int oracle_strassen(int transA, int transB, int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int dtype,
                    int depth, int variant, double* out) {
    if (depth < 0 || variant < 0 || variant > 1) return -1;
    int64_t q = (int64_t)1 << depth;
    if (M % q || N % q || K % q) return -1;
    blk_t Ad = blk_alloc(M, K), Bd = blk_alloc(K, N);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            AT(Ad, i, k) = oracle_decode(transA ? A[k * lda + i] : A[i * lda + k], dtype);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            AT(Bd, k, j) = oracle_decode(transB ? B[j * ldb + k] : B[k * ldb + j], dtype);
    blk_t C = {out, M, N, N};
    strassen_rec(C, Ad, Bd, depth, variant);
    free(Ad.p); free(Bd.p);
    return 0;
}

/* The same recursion on dense fp64 matrices (used for the integer identity pins). */
int oracle_strassen_f64(int64_t M, int64_t N, int64_t K, const double* A, const double* B,
                        int depth, int variant, double* out) {
    if (depth < 0 || variant < 0 || variant > 1) return -1;
    int64_t q = (int64_t)1 << depth;
    if (M % q || N % q || K % q) return -1;
    blk_t Ad = blk_alloc(M, K), Bd = blk_alloc(K, N);
    memcpy(Ad.p, A, sizeof(double) * M * K);
    memcpy(Bd.p, B, sizeof(double) * K * N);
    blk_t C = {out, M, N, N};
    strassen_rec(C, Ad, Bd, depth, variant);
    free(Ad.p); free(Bd.p);
    return 0;
}

/* Naive triple loop on fp64 (used to pin the blocked, threaded loop above). */
void oracle_naive_f64(int64_t M, int64_t N, int64_t K, const double* A, const double* B,
                      double* out) {
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += A[i * K + k] * B[k * N + j];
            out[i * N + j] = s;
        }
}

/* Seven S69 products of one 2x2-blocked level for inspection (M1..M7), fp64. */
int oracle_s69_products(int64_t n, const double* A, const double* B, double* Mout) {
    if (n % 2) return -1;
    int64_t h = n / 2;
    blk_t Ad = {(double*)A, n, n, n}, Bd = {(double*)B, n, n, n};
    blk_t A11 = blk_sub(Ad, 0, 0), A12 = blk_sub(Ad, 0, 1), A21 = blk_sub(Ad, 1, 0), A22 = blk_sub(Ad, 1, 1);
    blk_t B11 = blk_sub(Bd, 0, 0), B12 = blk_sub(Bd, 0, 1), B21 = blk_sub(Bd, 1, 0), B22 = blk_sub(Bd, 1, 1);
    blk_t L = blk_alloc(h, h), R = blk_alloc(h, h), tmp = blk_alloc(h, h);
    blk_t out[7];
    for (int t = 0; t < 7; ++t) { blk_t b = {Mout + t * h * h, h, h, h}; out[t] = b; }
    blk_axpy(L, A11, A22, 1); blk_axpy(R, B11, B22, 1); classical(out[0], L, R);
    blk_axpy(L, A21, A22, 1); classical(out[1], L, B11);
    blk_axpy(R, B12, B22, -1); classical(out[2], A11, R);
    blk_axpy(R, B21, B11, -1); classical(out[3], A22, R);
    blk_axpy(L, A11, A12, 1); classical(out[4], L, B22);
    blk_axpy(L, A21, A11, -1); blk_axpy(R, B11, B12, 1); classical(out[5], L, R);
    blk_axpy(L, A12, A22, -1); blk_axpy(R, B21, B22, 1); classical(out[6], L, R);
    (void)blk_copy;
    free(L.p); free(R.p); free(tmp.p);
    return 0;
}

/* ---------------------------------------------------------------------------
 * 8-bit floating point (CS336 Lecture 05 notes, Page 27: FP8 E4M3 = 1 sign, 4
 * exponent, 3 mantissa bits; E5M2 = 1 sign, 5 exponent, 2 mantissa bits; a value
 * is stored as q = cast(x / s) and used as s * q; MXFP8 keeps one E8M0 scale per
 * block of 32 values).  The encodings are the OCP 8-bit formats:
 *   E4M3: bias 7, subnormals at exponent field 0, no infinities; S.1111.111 is NaN,
 *         so the largest finite value is 1.75 * 2^8 = 448.
 *   E5M2: bias 15, IEEE-style: exponent field 31 is infinity (fraction 0) or NaN.
 *   E8M0: an unsigned power of two, 2^(e - 127); e = 255 is NaN.
 * ------------------------------------------------------------------------- */
#define OR_E4M3 0
#define OR_E5M2 1
#define OR_E2M1 2   /* 4-bit values, two per byte (see oracle_gemm_f8) */

double oracle_decode_f8(uint8_t h, int fmt) {
    int sign = (h >> 7) & 1;
    int ebits = fmt == OR_E4M3 ? 4 : 5;
    int fbits = fmt == OR_E4M3 ? 3 : 2;
    int bias = fmt == OR_E4M3 ? 7 : 15;
    int emax = (1 << ebits) - 1;
    int e = (h >> fbits) & emax;
    int f = h & ((1 << fbits) - 1);
    double v;
    if (fmt == OR_E4M3 && e == emax && f == (1 << fbits) - 1) {
        v = NAN;                                   /* the only E4M3 NaN pattern */
    } else if (fmt == OR_E5M2 && e == emax) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, 1 - bias - fbits);    /* subnormal */
    } else {
        v = ldexp((double)((1 << fbits) | f), e - bias - fbits);
    }
    return sign ? -v : v;
}

double oracle_decode_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* 4-bit floating point (CS336 Lecture 05 notes, Page 29, "Frontiers in low
 * precision - MXFP4": the representable values are 0, +-0.5, +-1, +-1.5, +-2, +-3,
 * +-4, +-6, used with a block scale).  The code is the OCP E2M1 layout that gives
 * exactly that set: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa; exponent
 * field 0 is subnormal (0 or 0.5); no infinities or NaN.  Only the low nibble of
 * `h` is read. */
double oracle_decode_f4(uint8_t h) {
    int sign = (h >> 3) & 1;
    int e = (h >> 1) & 3;
    int f = h & 1;
    double v = e == 0 ? 0.5 * f : ldexp(1.0 + 0.5 * f, e - 1);
    return sign ? -v : v;
}

/* Value k of a row that starts at `row`: a byte for the 8-bit formats; for E2M1,
 * value k sits in byte k/2, in its low nibble when k is even and its high nibble
 * when k is odd (the OCP packing of two 4-bit values per byte). */
static double lp_value(const uint8_t* row, int64_t k, int fmt) {
    if (fmt == OR_E2M1) return oracle_decode_f4((uint8_t)(row[k / 2] >> (4 * (k & 1))));
    return oracle_decode_f8(row[k], fmt);
}

typedef struct {
    int64_t K, N;
    const double* Ad;     /* decoded, scaled rows of A: nrows x K */
    const double* Bd;     /* decoded, scaled op(B): K x N */
    double* H;            /* nrows x N */
    int64_t r0, r1;
} f8_job_t;

static void* f8_worker(void* p) {
    f8_job_t* J = (f8_job_t*)p;
    int64_t K = J->K, N = J->N;
    for (int64_t r = J->r0; r < J->r1; ++r) {
        const double* arow = J->Ad + r * K;
        double* hrow = J->H + r * N;
        for (int64_t j = 0; j < N; ++j) hrow[j] = 0.0;
        for (int64_t jb = 0; jb < N; jb += OR_JB) {   /* ascending k per element */
            int64_t je = jb + OR_JB < N ? jb + OR_JB : N;
            for (int64_t k = 0; k < K; ++k) {
                double a = arow[k];
                const double* brow = J->Bd + k * N;
                for (int64_t j = jb; j < je; ++j) hrow[j] += a * brow[j];
            }
        }
    }
    return NULL;
}

/*
 * oracle_gemm_f8: the 8-bit and 4-bit GEMM, all in fp64 from the exact values.
 *   A is M x K row-major (lda), B is N x K row-major (ldb): op(B) = B^T, both
 *   operands K-contiguous, as the quantized layouts of the notes' Page 27-28 keep
 *   them.  fmtA / fmtB: OR_E4M3, OR_E5M2 (one byte a value, lda/ldb in values =
 *   bytes) or OR_E2M1 (two values a byte as lp_value reads them, lda/ldb in bytes,
 *   K even).  Each operand value is used as s * q (Page 27; Page 29 for 4-bit):
 *     s = the per-tensor scale (scale_a, scale_b) when the block-scale array is
 *         NULL, else the E8M0 scale of the value's block of 32 along K:
 *         sA(i,k) = mxA[i * ldmxA + k / 32], sB(j,k) = mxB[j * ldmxB + k / 32].
 *   D[i][j] = alpha * sum_k sA(i,k) qA[i][k] * sB(j,k) qB[j][k]
 *             + beta * C_in[i][j] + bias[j]          (k ascending)
 *   Q = RNE of D to the 16-bit output type; ss[r] = sum_j Q^2 with ROWSUMSQ.
 *   Outputs for the selected rows as in oracle_gemm.  Returns -1 on bad arguments.
 */
int oracle_gemm_f8(int64_t M, int64_t N, int64_t K, double alpha, const uint8_t* A,
                   int64_t lda, int fmtA, const uint8_t* B, int64_t ldb, int fmtB,
                   double scale_a, double scale_b, const uint8_t* mxA, int64_t ldmxA,
                   const uint8_t* mxB, int64_t ldmxB, double beta, const uint16_t* Cin,
                   int64_t ldc, int dtype, int epi, const uint16_t* bias, const int64_t* rows,
                   int64_t nrows, double* D, uint16_t* Q, double* ss, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return -1;
    if (fmtA < OR_E4M3 || fmtA > OR_E2M1 || fmtB < OR_E4M3 || fmtB > OR_E2M1) return -1;
    if ((fmtA == OR_E2M1 || fmtB == OR_E2M1) && K % 2) return -1;
    if ((mxA || mxB) && K % 32) return -1;
    if (epi & ~(OR_EPI_BIAS | OR_EPI_ROWSUMSQ)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    double* Ad = (double*)malloc(sizeof(double) * (nrows * K > 0 ? nrows * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (K * N > 0 ? K * N : 1));
    double* H = (double*)malloc(sizeof(double) * (nrows * N > 0 ? nrows * N : 1));
    if (!Ad || !Bd || !H) { free(Ad); free(Bd); free(H); return -1; }
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t i = rows[r];
            const double s = mxA ? oracle_decode_e8m0(mxA[i * ldmxA + k / 32]) : scale_a;
            Ad[r * K + k] = s * lp_value(A + i * lda, k, fmtA);
        }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) {
            const double s = mxB ? oracle_decode_e8m0(mxB[j * ldmxB + k / 32]) : scale_b;
            Bd[k * N + j] = s * lp_value(B + j * ldb, k, fmtB);
        }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    f8_job_t jobs[256];
    int64_t per = (nrows + nthreads - 1) / nthreads;
    int launched = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = t * per, r1 = r0 + per < nrows ? r0 + per : nrows;
        if (r0 >= r1) break;
        f8_job_t j = {K, N, Ad, Bd, H, r0, r1};
        jobs[t] = j;
        pthread_create(&th[t], NULL, f8_worker, &jobs[t]);
        ++launched;
    }
    for (int t = 0; t < launched; ++t) pthread_join(th[t], NULL);
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        double sum_sq = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double d = alpha * H[r * N + j];
            if (beta != 0.0) d += beta * oracle_decode(Cin[i * ldc + j], dtype);
            if (epi & OR_EPI_BIAS) d += oracle_decode(bias[j], dtype);
            D[r * N + j] = d;
            uint16_t q = oracle_encode(d, dtype);
            Q[r * N + j] = q;
            double w = oracle_decode(q, dtype);
            sum_sq += w * w;
        }
        if ((epi & OR_EPI_ROWSUMSQ) && ss) ss[r] = sum_sq;
    }
    free(Ad); free(Bd); free(H);
    return 0;
}

/* ---------------------------------------------------------------------------
 * MX quantization (CS336 Lecture 05 notes, Page 27: a value is stored as
 * q = cast(x / s) and used as s * q, the scale bringing the values into the
 * format's range; MX keeps one E8M0 scale per block of 32 values; Pages 27-28:
 * block scales make a transpose nontrivial, so the transposed operand is quantized
 * on its own, its blocks running along the other dimension).  Readings:
 *   s = 2^e, e the smallest integer with amax <= maxval * 2^e (maxval the format's
 *   largest finite value: E4M3 448, E5M2 57344, E2M1 6), clamped to [-127, 127];
 *   an all-zero block gets e = 0 (scale byte 127);
 *   q = the format's finite value nearest to x / s, ties to the code with the even
 *   last bit, the sign of x kept (a negative value that rounds to 0 gives -0).
 * ------------------------------------------------------------------------- */
static double lp_code_value(int code, int fmt) {
    return fmt == OR_E2M1 ? oracle_decode_f4((uint8_t)code) : oracle_decode_f8((uint8_t)code, fmt);
}

/* The nonnegative finite codes of a format in increasing value order (codes with the
 * sign bit clear; E4M3's NaN pattern and E5M2's infinities and NaNs left out). */
static int lp_positive_codes(int fmt, int* codes) {
    int n = 0, top = fmt == OR_E2M1 ? 8 : 128;
    for (int c = 0; c < top; ++c) {
        double v = lp_code_value(c, fmt);
        if (isfinite(v)) codes[n++] = c;
    }
    return n;   /* values increase with the code for sign-magnitude formats */
}

static int lp_round(double v, int fmt, const int* pos, int npos) {
    int sign = signbit(v) ? 1 : 0;
    double a = fabs(v);
    int lo = 0, hi = npos - 1;              /* largest code with value <= a */
    if (a >= lp_code_value(pos[hi], fmt)) {
        lo = hi;
    } else {
        while (hi - lo > 1) {
            int mid = (lo + hi) / 2;
            if (lp_code_value(pos[mid], fmt) <= a) lo = mid; else hi = mid;
        }
    }
    int c = pos[lo];
    if (lo + 1 < npos) {
        double dl = a - lp_code_value(pos[lo], fmt);
        double dh = lp_code_value(pos[lo + 1], fmt) - a;
        if (dh < dl || (dh == dl && (pos[lo + 1] & 1) == 0)) c = pos[lo + 1];
    }
    int sbit = fmt == OR_E2M1 ? 8 : 128;
    return sign ? (c | sbit) : c;
}

int oracle_quantize_mx(const uint16_t* X, int64_t rows, int64_t cols, int64_t ldx, int dtype,
                       int fmt, int transpose, uint8_t* Q, int64_t ldq, uint8_t* S,
                       int64_t lds) {
    if (rows < 0 || cols < 0 || fmt < OR_E4M3 || fmt > OR_E2M1) return -1;
    const int64_t orows = transpose ? cols : rows;   /* rows of the quantized matrix */
    const int64_t olen = transpose ? rows : cols;    /* values in each of its rows */
    if (olen % 32) return -1;
    const double maxval = fmt == OR_E4M3 ? 448.0 : fmt == OR_E5M2 ? 57344.0 : 6.0;
    int pos[128];
    const int npos = lp_positive_codes(fmt, pos);
    for (int64_t r = 0; r < orows; ++r) {
        for (int64_t b = 0; b < olen / 32; ++b) {
            double x[32], amax = 0.0;
            for (int t = 0; t < 32; ++t) {
                const int64_t k = 32 * b + t;
                const uint16_t h = transpose ? X[k * ldx + r] : X[r * ldx + k];
                x[t] = oracle_decode(h, dtype);
                if (!isfinite(x[t])) return -1;
                if (fabs(x[t]) > amax) amax = fabs(x[t]);
            }
            int e = 0;
            if (amax > 0.0) {
                e = (int)ceil(log2(amax / maxval));
                while (amax > ldexp(maxval, e)) ++e;          /* exact: smallest such e */
                while (amax <= ldexp(maxval, e - 1)) --e;
            }
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            S[r * lds + b] = (uint8_t)(e + 127);
            for (int t = 0; t < 32; ++t) {
                const int64_t k = 32 * b + t;
                const int c = lp_round(ldexp(x[t], -e), fmt, pos, npos);
                if (fmt == OR_E2M1) {
                    uint8_t* p = Q + r * ldq + k / 2;
                    *p = (k & 1) ? (uint8_t)((*p & 0x0F) | (c << 4)) : (uint8_t)((*p & 0xF0) | c);
                } else {
                    Q[r * ldq + k] = (uint8_t)c;
                }
            }
        }
    }
    return 0;
}
