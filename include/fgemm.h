/*
 * fgemm.h — C ABI of libfgemm: half-precision GEMM for AMD MI355X (gfx950).
 *
 *   C = alpha * op(A) * op(B) + beta * C      fp16 or bf16 in, fp32 accumulate
 *
 * The operation is the HGEMM of the CUDA-L2 abstract (chatpaper.ai page, NN and TN
 * layouts); 16-bit inputs with wider accumulation follow CS336 Lecture 05 notes,
 * Page 26.  Two paths compute it:
 *   - classical: a tiled MFMA GEMM whose epilogue (scale, beta*C, bias, row
 *     statistics, activation) runs before the store (PingPong GEMM note on
 *     tilnote.io: mainloop + epilogue; CODA section: RMSNorm statistics in the
 *     first GEMM's epilogue, scaling and SwiGLU in the second's);
 *   - Strassen/Winograd: one or two levels of the 2x2 block recursion with seven
 *     sub-products per level (FalconGEMM summary on euno.news, Methodology 1, 3).
 * An analytic model picks the path per shape from compute throughput, memory
 * bandwidth and the per-level addition traffic (FalconGEMM summary, Methodology 4
 * and 5; roofline of CS336 Lecture 05 notes, Page 21; tile and wave quantization,
 * Pages 43 and 48).
 *
 * Conventions for every entry point:
 *   - Storage is row-major.  op = N: A is M x K (lda >= K); op = T: A is stored
 *     K x M (lda >= M).  op = N: B is K x Nb (ldb >= Nb); op = T: B is stored
 *     Nb x K (ldb >= K).  Nb = N, or 2*N with FGEMM_EPI_RMS_SWIGLU.  C is M x N
 *     with ldc >= N.  Leading dimensions are in elements.
 *   - A, B, C, the epilogue vectors and the workspace are DEVICE pointers owned by
 *     the caller; the library never frees them.  alpha and beta are host floats.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = the null stream) and the
 *     call returns after the enqueue; nothing is synchronised.
 *   - beta == 0: C is never read (NaN or Inf in C do not propagate).
 *   - M == 0 or N == 0: nothing is done.  K == 0: C = beta*C (+ epilogue).
 *   - C must not overlap A or B.  C may be read and written in place (beta*C).
 *   - Arguments are validated before any device work; errors are returned
 *     synchronously and nothing is enqueued.  No C++ exception crosses the ABI.
 *   - A handle is not thread safe: use one per host thread.  Calls that overlap
 *     on one handle's workspace must be on one stream.
 *   - Fast path: 16-byte aligned pointers and leading dimensions that are
 *     multiples of 8; anything else runs a correct element-wise path.
 */
#ifndef FGEMM_H
#define FGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fgemm_handle_s* fgemm_handle_t;

typedef enum {
    FGEMM_OK = 0,
    FGEMM_ERR_INVALID_VALUE = 1, /* a bad size, leading dimension, pointer or flag   */
    FGEMM_ERR_NOT_SUPPORTED = 2, /* a valid request this library does not implement  */
    FGEMM_ERR_WORKSPACE = 3,     /* a forced plan needs more workspace than is set   */
    FGEMM_ERR_ALLOC = 4,         /* a device allocation failed                       */
    FGEMM_ERR_HIP = 5            /* a HIP runtime or launch error                    */
} fgemm_status_t;

typedef enum { FGEMM_OP_N = 0, FGEMM_OP_T = 1 } fgemm_op_t;

/* A, B and C share the type; accumulation is fp32. */
typedef enum { FGEMM_F16 = 0, FGEMM_BF16 = 1 } fgemm_dtype_t;

/* Epilogue flags (tilnote.io PingPong GEMM note: GEMM = mainloop + epilogue; CODA
 * section: norm statistics in the first GEMM's epilogue, scaling and SwiGLU in the
 * second's).  Per output element, in this order:
 *   D = alpha*acc + beta*C + bias[j]             (BIAS adds bias[j])
 *   C[i][j] = RNE16(D)
 *   ROWSUMSQ: rowsumsq[i] = sum_j C[i][j]^2 of the rounded, written row (fp32).
 * RMS_SWIGLU (alone): op(B) has 2N columns, gate = columns [0, N), up = [N, 2N):
 *   r_i = 1/sqrt(rms_rowsumsq[i]/rms_n + rms_eps)
 *   g = r_i*alpha*acc_gate, u = r_i*alpha*acc_up,
 *   C[i][j] = RNE16(silu(g)*u + beta*C[i][j]),  silu(x) = x/(1+exp(-x)).
 * ACT (with BIAS and ROWSUMSQ, not with ROPE): D = act(D) before the rounding;
 *   act is ReLU, SiLU, or GELU in the tanh form of Hendrycks and Gimpel,
 *   0.5x(1 + tanh(sqrt(2/pi)(x + 0.044715x^3))).
 * ROPE (with BIAS and ROWSUMSQ, not with ACT; same note, CODA section: RoPE in the
 *   epilogue): the rotary embedding of Su et al. (RoFormer) on interleaved pairs
 *   before the rounding.  Column j is at d = j % rope_head_dim of its head; pair
 *   (2p, 2p+1), p = d/2, of row i turns by theta = pos_i * rope_theta^(-2p/rope_head_dim):
 *     D[i][2p] <- D[i][2p] cos(theta) - D[i][2p+1] sin(theta)
 *     D[i][2p+1] <- D[i][2p] sin(theta) + D[i][2p+1] cos(theta)
 *   with pos_i = rope_positions[i], or i + rope_offset when rope_positions is NULL.
 *   (The half-split pairing (d, d + hd/2) is this one after a fixed permutation
 *   of op(B)'s columns within each head.)
 * SWIGLU_BWD (alone; same note, CODA section: backward passes of SwiGLU in the
 *   epilogue): the backward of RMS_SWIGLU with the row scale held fixed.  op(B)
 *   has the forward's 2N columns [gate | up]; g, u and r_i are as in RMS_SWIGLU;
 *   dO = swiglu_dout[i][j] (device, M x N, leading dimension swiglu_ldd) is the
 *   incoming gradient.  C is M x 2N (ldc >= 2N), the gradient with respect to
 *   op(A)op(B):
 *     C[i][j]     = RNE16(dO * u * silu'(g) * r_i * alpha)
 *     C[i][N + j] = RNE16(dO * silu(g) * r_i * alpha),
 *   silu'(x) = s(x)(1 + x(1 - s(x))), s(x) = 1/(1+exp(-x)); beta must be 0.
 *   With rms_grad != NULL it also writes the gradient with respect to each row's
 *   scale: rms_grad[i] = sum_j dO (silu'(g) g u + silu(g) u) / r_i  (fp32, [M]).
 * RMS_BWD (alone; the rest of the RMSNorm backward): with r_i = 1/sqrt(ss_i/n + eps)
 *   from rms_rowsumsq, rms_n, rms_eps and the scale gradient rms_grad[i] (input),
 *   C[i][j] = RNE16(alpha*acc + c_i * X[i][j]),  c_i = -r_i^3 * rms_grad[i] / n,
 *   X = rms_x (device, M x N 16-bit, leading dimension rms_ldx), the normalised
 *   layer's input; beta must be 0.  For the chain Y -> RMS scale -> Y W2 -> SwiGLU:
 *   dH from SWIGLU_BWD, then dY = dH W2^T with RMS_BWD and X = Y. */
enum {
    FGEMM_EPI_NONE = 0,
    FGEMM_EPI_BIAS = 1,
    FGEMM_EPI_ROWSUMSQ = 2,
    FGEMM_EPI_RMS_SWIGLU = 4,
    FGEMM_EPI_ACT = 8,
    FGEMM_EPI_ROPE = 16,
    FGEMM_EPI_SWIGLU_BWD = 32,
    FGEMM_EPI_RMS_BWD = 64
};
typedef enum { FGEMM_ACT_RELU = 1, FGEMM_ACT_SILU = 2, FGEMM_ACT_GELU_TANH = 3 } fgemm_act_t;

typedef struct {
    uint32_t flags;             /* FGEMM_EPI_* bits                                  */
    const void* bias;           /* BIAS: device [N], same 16-bit type as C           */
    float* rowsumsq;            /* ROWSUMSQ: device [M] fp32 output                  */
    const float* rms_rowsumsq;  /* RMS_SWIGLU, SWIGLU_BWD, RMS_BWD: device [M] fp32
                                   sums of squares of the normalised rows (input)    */
    int64_t rms_n;              /* the same: width the statistics were taken over    */
    float rms_eps;              /* the same: epsilon inside the square root          */
    int32_t act;                /* ACT: fgemm_act_t                                   */
    const int32_t* rope_positions; /* ROPE: device [M] positions, or NULL            */
    int64_t rope_offset;        /* ROPE: position of row 0 when rope_positions is NULL */
    int64_t rope_head_dim;      /* ROPE: divides N; a multiple of 8, at most 1024
                                   (other even widths: FGEMM_ERR_NOT_SUPPORTED)     */
    float rope_theta;           /* ROPE: frequency base (> 0), e.g. 10000             */
    const void* swiglu_dout;    /* SWIGLU_BWD: device [M][swiglu_ldd] 16-bit gradient */
    int64_t swiglu_ldd;         /* SWIGLU_BWD: leading dimension of swiglu_dout (>= N) */
    float* rms_grad;            /* SWIGLU_BWD: device [M] output, or NULL;
                                   RMS_BWD: device [M] input                          */
    const void* rms_x;          /* RMS_BWD: device [M][rms_ldx] 16-bit                */
    int64_t rms_ldx;            /* RMS_BWD: leading dimension of rms_x (>= N)         */
} fgemm_epilogue_t;

typedef enum {
    FGEMM_PATH_CLASSICAL = 0,
    FGEMM_PATH_STRASSEN = 1
} fgemm_path_t;

/* Strassen (1969): 7 products, 18 block additions.
 * Winograd form: 7 products, 15 block additions (8 pre-add outputs instead of 10).
 * R223: a rectangular block scheme <2,2,3;11> (FalconGEMM summary, Methodology 1:
 * the catalog's tensor-decomposition schemes): op(A) in 2 x 2 blocks, op(B) and C
 * in 2 x 3, eleven block products (twelve classically): Strassen (1969) on the
 * first two column blocks of op(B) and C, the four block products of the third.
 * Depth 1 only; M and K multiples of 32, N a multiple of 48; epilogues NONE and
 * BIAS (others FGEMM_ERR_NOT_SUPPORTED). */
typedef enum {
    FGEMM_VARIANT_S69 = 0,
    FGEMM_VARIANT_WINOGRAD = 1,
    FGEMM_VARIANT_R223 = 2
} fgemm_variant_t;

/* A plan: what fgemm_select chose (or what a caller forces through fgemm_gemm_plan). */
typedef struct {
    int32_t path;               /* fgemm_path_t                                       */
    int32_t depth;              /* Strassen recursion depth, 1 or 2 (0 = classical)  */
    int32_t variant;            /* fgemm_variant_t                                    */
    int32_t tile_m, tile_n, tile_k; /* macro-tile of the classical kernel (products) */
    int32_t split_k;            /* K-splits of the classical kernel (1 = none)        */
    size_t workspace_bytes;     /* device workspace the plan needs                    */
    double t_pred_us;           /* model time of this plan                            */
    double t_classical_pred_us; /* model time of the best classical plan              */
    double pred_rel_err;        /* predicted normwise error of the plan against the
                                   exactly rounded result, from calibrated per-path
                                   figures on i.i.d. inputs (FalconGEMM summary,
                                   Methodology 4: accuracy guides the choice); not a
                                   worst-case bound                                  */
} fgemm_plan_t;

/* Constants of the analytic model.  fgemm_create fills them from the device and
 * the built-in calibration; fgemm_set_model replaces them. */
typedef struct {
    int32_t compute_units;      /* CUs that run workgroups                            */
    double peak_tflops;         /* dense 16-bit MFMA peak, TFLOP/s                    */
    double hbm_gbps;            /* HBM bandwidth, GB/s                                */
    double eta_mfma;            /* fraction of MFMA peak a full tile wave reaches     */
    double eta_hbm;             /* fraction of HBM bandwidth streaming kernels reach  */
    double launch_us;           /* per-kernel launch and drain cost, microseconds     */
    double max_workspace_bytes; /* AUTO never plans above this workspace (default a
                                   third of the device's memory)                     */
    double max_rel_err;         /* AUTO never plans a path whose predicted normwise
                                   error ||C - RNE(D)||_F / ||RNE(D)||_F exceeds this
                                   (default 5e-3); see fgemm_plan_t.pred_rel_err     */
} fgemm_model_t;

/* Handle: reads the device's CU count and architecture; fails with
 * FGEMM_ERR_NOT_SUPPORTED on anything but gfx950 and FGEMM_ERR_HIP without a device.
 * Calls through a handle run on its device (made current for the call, the caller's
 * current device restored on return); their streams and pointers must belong to it. */
fgemm_status_t fgemm_create(fgemm_handle_t* handle, int device);
fgemm_status_t fgemm_destroy(fgemm_handle_t handle);

/* Caller-owned device workspace (for example a torch tensor).  Without one the
 * handle allocates what a plan needs with hipMalloc and keeps it until destroyed:
 * for automatic plans up to model.max_workspace_bytes (by default a third of the
 * device's memory; Strassen at 49152^3 takes 42 GB).  With one, automatic plans
 * stay within its size and NULL (bytes 0) returns to the handle's own. */
fgemm_status_t fgemm_set_workspace(fgemm_handle_t handle, void* dptr, size_t bytes);

fgemm_status_t fgemm_get_model(fgemm_handle_t handle, fgemm_model_t* model);
fgemm_status_t fgemm_set_model(fgemm_handle_t handle, const fgemm_model_t* model);

/* The model's pick for a shape: the plan of least predicted time among the
 * classical kernel and Strassen/Winograd at depth 1 and 2, subject to the
 * accuracy (model.max_rel_err against the plan's pred_rel_err), divisibility,
 * epilogue and workspace guards; a tighter error budget lowers the depth or keeps
 * the classical path.  With ROWSUMSQ a statistics guard also applies: a row's sum
 * of squares moves by up to about twice the output's relative error, so such calls
 * go to Strassen only where 2*pred_rel_err <= 1e-3 (with the built-in error table:
 * never; the statistics then stay within 1e-3 on every automatic plan).  Host only;
 * it caches nothing (fgemm_gemm keeps its own pick per shape in the handle). */
fgemm_status_t fgemm_select(fgemm_handle_t handle, fgemm_op_t transA, fgemm_op_t transB,
                            int64_t M, int64_t N, int64_t K, fgemm_dtype_t dtype,
                            const fgemm_epilogue_t* epilogue, fgemm_plan_t* plan);

/* The same decision as a pure function of an explicit model (no handle, no GPU). */
fgemm_status_t fgemm_select_model(const fgemm_model_t* model, fgemm_op_t transA,
                                  fgemm_op_t transB, int64_t M, int64_t N, int64_t K,
                                  fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                                  fgemm_plan_t* plan);

/* C = alpha*op(A)*op(B) + beta*C with the epilogue (NULL = none), on the plan
 * fgemm_select picks.  Without a caller workspace, if hipMalloc cannot hold the
 * workspace that plan needs, the call plans again within what the handle already
 * holds (at worst the classical path) and keeps that plan for the shape;
 * FGEMM_ERR_ALLOC only when even that fails.  Nothing is enqueued before the
 * workspace is in hand.  Once a call of the same shape has sized the workspace, a
 * call only enqueues kernels (no allocation, memset or synchronisation), so it can
 * be captured into a HIP graph. */
fgemm_status_t fgemm_gemm(fgemm_handle_t handle, fgemm_op_t transA, fgemm_op_t transB,
                          int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                          int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                          int64_t ldc, fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                          void* stream);

/* The same on an explicit plan (path, depth, variant).  Tile fields of 0 let the
 * library choose.  Strassen needs M, K and the column count of op(B) (N, or 2N
 * with RMS_SWIGLU) divisible by 8*2^depth and aligned operands, else
 * FGEMM_ERR_NOT_SUPPORTED; too small a caller workspace gives FGEMM_ERR_WORKSPACE.
 * On the Strassen path the epilogues run in the top-level block post-add (all but
 * SWIGLU_BWD and RMS_BWD, which are classical only): with RMS_SWIGLU the 2x2 split
 * of op(B)'s 2N columns is exactly the gate/up boundary, so gate and up of one
 * output meet in the same post-add lane. */
fgemm_status_t fgemm_gemm_plan(fgemm_handle_t handle, const fgemm_plan_t* plan,
                               fgemm_op_t transA, fgemm_op_t transB, int64_t M, int64_t N,
                               int64_t K, float alpha, const void* A, int64_t lda,
                               const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                               fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                               void* stream);

/* 8-bit floating-point formats of fgemm_gemm_f8 (the OCP encodings): E4M3 is
 * 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities, largest finite
 * 448; E5M2 is 1 sign, 5 exponent (bias 15) and 2 mantissa bits, IEEE-style
 * infinities and NaNs, largest finite 57344 (CS336 Lecture 05 notes, Page 27). */
typedef enum { FGEMM_E4M3 = 0, FGEMM_E5M2 = 1, FGEMM_E2M1 = 2 } fgemm_f8_format_t;
/* FGEMM_E2M1 (the 4-bit format of fgemm_gemm_mxf4) is taken by fgemm_quantize_mx
 * only; fgemm_gemm_f8 and fgemm_gemm_mxf8 refuse it. */

/* 8-bit GEMM with per-tensor scales (CS336 Lecture 05 notes, Page 27: a value is
 * stored as q = cast(x/s) and used as s*q, one fp32 scale per tensor; Page 28:
 * transposes are quantized separately, so both operands arrive K-contiguous):
 *   C = alpha * (scale_a * A) * (scale_b * B)^T + beta * C
 * A is M x K row-major 8-bit codes (lda >= K bytes), B is N x K row-major (ldb >= K
 * bytes), each in its own format; C is M x N in the 16-bit type `dtype` (ldc >= N).
 * The products are exact and accumulate in fp32 (v_mfma_scale_f32_32x32x64_f8f6f4
 * with unit block scales); alpha*scale_a*scale_b is formed once and applied to the
 * fp32 sums, then beta*C and the epilogue: NONE, BIAS and ROWSUMSQ as in
 * fgemm_gemm (others FGEMM_ERR_NOT_SUPPORTED).  Needs K % 128 == 0, lda and ldb
 * multiples of 16, ldc a multiple of 8, 16-byte aligned A, B and C, and
 * alpha*scale_a*scale_b zero or a normal fp32 value, else FGEMM_ERR_NOT_SUPPORTED.
 * Pointers, streams, errors and beta = 0 as for fgemm_gemm; ROWSUMSQ partials use
 * the handle's workspace. */
fgemm_status_t fgemm_gemm_f8(fgemm_handle_t handle, int64_t M, int64_t N, int64_t K, float alpha,
                             const void* A, int64_t lda, fgemm_f8_format_t a_format,
                             float scale_a, const void* B, int64_t ldb,
                             fgemm_f8_format_t b_format, float scale_b, float beta, void* C,
                             int64_t ldc, fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                             void* stream);

/* MXFP8 GEMM: the 8-bit GEMM of fgemm_gemm_f8 with one E8M0 scale per block of 32
 * values along K instead of one scale per tensor (CS336 Lecture 05 notes, Page 27:
 * MXFP8 keeps an FP8 E8M0 scale, 2^(e-127), for every 32 values):
 *   C[i][j] = alpha * sum_k sA(i,k) A[i][k] * sB(j,k) B[j][k] + beta * C[i][j]
 *   sA(i,k) = 2^(a_scales[i*ld_a_scales + k/32] - 127), sB likewise from b_scales.
 * a_scales is M x (K/32) bytes, b_scales N x (K/32) bytes, row-major device arrays
 * (a leading dimension below K/32 is FGEMM_ERR_INVALID_VALUE); the leading
 * dimensions must be multiples of 16 of at least K/32 rounded up to a multiple of
 * 16 (the kernel reads 16 scales, four phases, per row at a time; the bytes past
 * K/32 are read and not used) and the arrays 16-byte aligned, else
 * FGEMM_ERR_NOT_SUPPORTED.  The MFMA applies each lane's block scale
 * (v_mfma_scale_f32_32x32x64_f8f6f4).  K = 0 reads no scale (the arrays may be
 * null); everything else is as for fgemm_gemm_f8. */
fgemm_status_t fgemm_gemm_mxf8(fgemm_handle_t handle, int64_t M, int64_t N, int64_t K,
                               float alpha, const void* A, int64_t lda,
                               fgemm_f8_format_t a_format, const void* a_scales,
                               int64_t ld_a_scales, const void* B, int64_t ldb,
                               fgemm_f8_format_t b_format, const void* b_scales,
                               int64_t ld_b_scales, float beta, void* C, int64_t ldc,
                               fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                               void* stream);

/* MXFP4 GEMM (CS336 Lecture 05 notes, Page 29: 4-bit floating point holds only 0,
 * +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6 and is usable only with block scales):
 *   C[i][j] = alpha * sum_k sA(i,k) qA(i,k) * sB(j,k) qB(j,k) + beta * C[i][j]
 * with q the E2M1 value (1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent field 0 gives 0 and 0.5) and s the E8M0 scale 2^(e-127) of the value's
 * block of 32 along K.  A is M x K values, B is N x K values, both row-major and
 * K-contiguous, packed two values a byte: value k of a row is the low nibble of
 * byte k/2 when k is even, its high nibble when k is odd.  lda and ldb are row
 * strides in BYTES (>= K/2); a_scales / b_scales, ld_a_scales / ld_b_scales as for
 * fgemm_gemm_mxf8.  The page's slide groups 16 values under an E4M3 scale; the
 * gfx950 block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, format E2M1) applies
 * E8M0 scales to blocks of 32, so the scales here are the OCP MX ones.  Needs
 * K % 256 == 0, lda and ldb multiples of 16, ldc a multiple of 8 and 16-byte
 * aligned A, B and C, else FGEMM_ERR_NOT_SUPPORTED; K = 0 reads no value or scale
 * (C = beta*C + bias).  Output type, epilogues (NONE, BIAS, ROWSUMSQ), pointers,
 * streams and errors as for fgemm_gemm_f8. */
fgemm_status_t fgemm_gemm_mxf4(fgemm_handle_t handle, int64_t M, int64_t N, int64_t K,
                               float alpha, const void* A, int64_t lda, const void* a_scales,
                               int64_t ld_a_scales, const void* B, int64_t ldb,
                               const void* b_scales, int64_t ld_b_scales, float beta, void* C,
                               int64_t ldc, fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue,
                               void* stream);

/* MX quantization for the 8-bit and 4-bit GEMMs (CS336 Lecture 05 notes, Page 27: a
 * value is stored as q = cast(x/s) and used as s*q, one E8M0 scale per block of 32;
 * Pages 27-28: block scales make a transpose nontrivial, so the transposed operand
 * is quantized separately, its blocks running along the other dimension).
 * X is rows x cols 16-bit values of `x_dtype`, row-major (ldx >= cols elements).
 *   transpose == 0: quantizes X itself: Q has `rows` rows of `cols` values, blocks of
 *     32 consecutive values of a row of X (cols % 32 == 0);
 *   transpose != 0: quantizes X^T: Q has `cols` rows of `rows` values, row j holding
 *     column j of X, blocks of 32 consecutive rows of X (rows % 32 == 0);
 * in both cases the K-contiguous layout the GEMMs take (A M x K, B N x K).  For a
 * block with largest magnitude amax, e is the smallest integer with
 * amax <= maxval * 2^e (maxval = 448 for E4M3, 57344 for E5M2, 6 for E2M1; clamped
 * to [-127, 127]; 0 for an all-zero block), scales[r*ld_scales + b] = e + 127, and
 * each value is coded as the format's value nearest to x * 2^-e, ties to the even
 * code, its sign kept.  Q holds one byte a value (E4M3, E5M2) or two values a byte
 * (E2M1, value 2i in the low nibble); ldq is its row stride in BYTES.  ld_scales
 * (bytes) >= the quantized row length / 32; only those bytes of a scale row are
 * written.  X, Q, scales are device pointers; work is enqueued on `stream`.  Needs X
 * and Q 16-byte aligned, ldx % 8 == 0, ldq % 16 == 0, else FGEMM_ERR_NOT_SUPPORTED;
 * a row length not a multiple of 32, ldq below a quantized row, ld_scales below its
 * block count, an unknown format or type, or a null pointer with work to do is
 * FGEMM_ERR_INVALID_VALUE.  Inputs are finite (NaN or Inf give unspecified codes). */
fgemm_status_t fgemm_quantize_mx(const void* X, int64_t rows, int64_t cols, int64_t ldx,
                                 fgemm_dtype_t x_dtype, int transpose, fgemm_f8_format_t format,
                                 void* Q, int64_t ldq, void* scales, int64_t ld_scales,
                                 void* stream);

/* Size of the fixed per-device scratch array behind fgemm_gemm_noalloc. */
#define FGEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The arguments, results
 * and errors of fgemm_gemm, on the classical path only (the model's classical
 * pick, split K included), with every scratch buffer its kernels use (the
 * row-statistics partials of ROWSUMSQ and SWIGLU_BWD, the fp32 split-K slices) in
 * a fixed device array of FGEMM_NOALLOC_SCRATCH_BYTES.  Each device holds its own
 * array from the first fgemm_create on it until the process ends.  The call makes
 * no device or host allocation: no hipMalloc or hipFree, and the handle's
 * workspace is never used or grown; its plans are kept in a fixed table in the
 * handle.  A call whose plan needs more scratch than the array holds returns
 * FGEMM_ERR_WORKSPACE before anything is enqueued.  Every call on a device shares
 * that device's array and leaves its contents there (no part of it needs to start
 * at zero): calls that may overlap in time on one device (different streams,
 * handles or host threads) race on it and must be serialised by the caller. */
fgemm_status_t fgemm_gemm_noalloc(fgemm_handle_t handle, fgemm_op_t transA, fgemm_op_t transB,
                                  int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                                  int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                                  int64_t ldc, fgemm_dtype_t dtype,
                                  const fgemm_epilogue_t* epilogue, void* stream);

/* Argument validation alone (pure; no handle, no device): the status fgemm_gemm
 * would return before enqueuing anything. */
fgemm_status_t fgemm_check_args(fgemm_op_t transA, fgemm_op_t transB, int64_t M, int64_t N,
                                int64_t K, const void* A, int64_t lda, const void* B,
                                int64_t ldb, float beta, const void* C, int64_t ldc,
                                fgemm_dtype_t dtype, const fgemm_epilogue_t* epilogue);

/* Tile quantization: ceil(M/tile_m) * ceil(N/tile_n) output tiles (CS336 Lecture
 * 05 notes, Page 43: 256/128 gives 2 tiles per dimension, 257/128 gives 3). */
int64_t fgemm_tile_count(int64_t M, int64_t N, int64_t tile_m, int64_t tile_n);

/* Wave quantization: waves = ceil(tiles/units); *tail_fraction = share of the
 * units busy in the last wave (CS336 Lecture 05 notes, Page 48: 98 tiles on 108
 * units is one wave; 120 tiles is two, the second 12/108 busy). */
int64_t fgemm_wave_count(int64_t tiles, int64_t units, double* tail_fraction);

/* The error model behind the accuracy guard (pure): the predicted normwise error
 * ||C - RNE(D)||_F / ||RNE(D)||_F of `plan` (classical, or Strassen/Winograd at its
 * depth and variant) for 16-bit inputs of type `dtype`; negative for an invalid
 * dtype, path, depth or variant.  Calibrated on MI355X with i.i.d. inputs; not a
 * worst-case bound. */
double fgemm_plan_rel_err(fgemm_dtype_t dtype, const fgemm_plan_t* plan);

/* Read-bandwidth reference for the rooflines of the HBM-bound kernels (the decode
 * shapes, the Strassen additions): one streaming pass over `bytes` of device memory
 * at `src` with FGEMM_READ_PROBE_GROUPS workgroups of 256 threads, each over one
 * contiguous chunk with 16 independent 16-byte loads per thread in flight, enqueued
 * on `stream` (a hipStream_t; null is the default stream).  out[g] (device memory,
 * FGEMM_READ_PROBE_GROUPS words, written in full) receives the XOR of the 32-bit
 * words of chunk g, so the XOR of all of out is the XOR of every 32-bit word of src.
 * FGEMM_ERR_INVALID_VALUE for bytes < 0, bytes not a multiple of 16, a null out, or
 * (bytes > 0) a null or not 16-byte aligned src; FGEMM_ERR_HIP for a failed launch.
 * Timed on the same buffer and cache state as a kernel, it gives the rate a plain
 * read of that size reaches on the device. */
#define FGEMM_READ_PROBE_GROUPS 1024
fgemm_status_t fgemm_read_probe(const void* src, int64_t bytes, uint32_t* out, void* stream);

const char* fgemm_status_string(fgemm_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FGEMM_H */
