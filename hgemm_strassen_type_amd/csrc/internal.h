// internal.h — declarations shared by the library's host code and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fgemm.h"

namespace fgemm {

// Element types of an operand as it sits in memory.
enum ElemType : int { kF16 = 0, kBF16 = 1 };
// 8-bit MFMA inputs: one code for the formats of both operands, fa and fb each
// 0 (E4M3) or 1 (E5M2), the MFMA's own format numbers.
constexpr int kF8Base = 4;
// Column width and wave columns of the 8-bit kernels' tile (row-statistics partials
// are [ceil(N / kF8TileN) * kF8WavesN][M]).
constexpr int kF8TileN = 256, kF8WavesN = 2;
constexpr int f8_code(int fa, int fb, int mx = 0) { return kF8Base + 4 * mx + 2 * fa + fb; }
// MXFP4: both operands E2M1, two values a byte, with E8M0 block scales (the same
// 8-bit-path kernel, a 4-bit operand mode).
constexpr int kF4MX = kF8Base + 8;

// MX quantization of a 16-bit matrix (dtype kF16/kBF16) into codes of format `fmt`
// (fgemm_f8_format_t) and E8M0 block scales, blocks along rows or, with transpose,
// along columns; arguments checked by the caller.
hipError_t launch_quantize_mx(const void* X, int64_t rows, int64_t cols, int64_t ldx, int dtype,
                              bool transpose, int fmt, void* Q, int64_t ldq, void* S, int64_t lds,
                              hipStream_t s);

// Epilogue kinds the kernel template is instantiated for.
enum EpiKind : int {
  kEpiStore16 = 0,   // 16-bit output: alpha, beta*C, optional bias, optional row sum of squares
  kEpiSwiGLU = 1,    // 16-bit output of silu(r*alpha*gate) * (r*alpha*up) + beta*C
  kEpiStore32 = 2,   // fp32 output of the raw accumulators (Strassen sub-products)
  kEpiAct = 3,       // kEpiStore16 plus an activation before rounding
  kEpiRope = 4,      // kEpiStore16 plus the rotary position embedding before rounding
  kEpiSwiGLUBwd = 5, // 16-bit gradient of the SwiGLU epilogue's input (2N columns)
  kEpiRmsBwd = 6,    // alpha*acc + c_i*X: the RMS scale's share of the input gradient
};

// Runtime epilogue switches inside kEpiStore16.
enum : uint32_t { kFlagBias = 1u, kFlagRowSumSq = 2u, kFlagBeta = 4u };

// One GEMM problem as the classical kernel sees it.  Pointers are device pointers.
// op(A) is M x K, op(B) is K x Nb (Nb = N, or 2N for SwiGLU), output M x N.
struct GemmProblem {
  const void* A;
  const void* B;
  void* C;              // output (16-bit or fp32)
  const void* Cin;      // beta*C input, same type/layout as C (may equal C)
  int64_t lda, ldb, ldc;
  int M, N, K;
  float alpha, beta;
  uint32_t flags;       // kFlag* bits
  const void* bias;     // [N] 16-bit
  float* ss_partial;    // [tiles_n * 2][M] per-wave-column partial sums of squares
  const float* rms_ss;  // [M] sums of squares for the RMS scale
  float rms_inv_n, rms_eps;
  int act;                  // kEpiAct: the activation
  int rope_hd;              // kEpiRope: head width (a multiple of 8, at most 1024)
  const int32_t* rope_pos;  // [M] positions, or null: row + rope_off
  int64_t rope_off;
  double rope_log2_base;
  const void* dout;         // kEpiSwiGLUBwd: [M][ldd] incoming 16-bit gradient
  int64_t ldd;
  // kEpiSwiGLUBwd: per-wave partials of the row-scale gradient (into ss_partial) when
  // set; kEpiRmsBwd: the row-scale gradient [M] (input) and X [M][ldx]
  int rms_grad_out;
  const float* rms_grad;
  const void* rms_x;
  int64_t ldx;
  // 8-bit MX inputs: E8M0 scales, one per 32 values along K, [M][ld_mxa] for A and
  // [N][ld_mxb] for B (bytes; rows hold whole 16-byte groups of 16 blocks)
  const void* mx_a;
  const void* mx_b;
  int64_t ld_mxa, ld_mxb;
};

// Up to 7 problems of one shape launched together (the Strassen sub-products).
// Work items are (problem, K slice, output tile) triples.  The launcher starts as
// many workgroups as the device holds at once (compute units x occupancy, capped
// by the item count); each loops over its share of the items.
struct GemmBatch {
  GemmProblem p[7];
  int count;
  int k_splits;   // kEpiStore32 only: K split into fp32 slices of M x ldc
  int cus;        // compute units of the device (0: one workgroup per item)
  int tiles;      // output tiles of the largest problem (set by the launcher)
};

// Kernel selection for one launch.
struct KernelKey {
  int tile;           // 0: 256x256, 1: 128x128, 2: 64x128 (skinny), 3: 32x128 (skinny)
  int a_kcontig;      // 1: op(A) rows are K-contiguous (A not transposed)
  int b_kcontig;      // 1: op(B) columns are K-contiguous (B transposed)
  int dtype;          // ElemType of the MFMA inputs and of 16-bit outputs
  int epi;            // EpiKind
  int vec;            // 1: 16-byte aligned fast path
  int odt;            // 8-bit inputs only: ElemType of the 16-bit output
};

// One instantiation unit per (MFMA dtype, A layout, B layout); each is compiled from
// gemm_inst.hip with its own -D switches.
#define FGEMM_INST_DECL(DT, AK, BK) \
  hipError_t launch_gemm_##DT##_##AK##BK(const KernelKey& k, const GemmBatch& b, hipStream_t s);
FGEMM_INST_DECL(0, 0, 0) FGEMM_INST_DECL(0, 0, 1) FGEMM_INST_DECL(0, 1, 0) FGEMM_INST_DECL(0, 1, 1)
FGEMM_INST_DECL(1, 0, 0) FGEMM_INST_DECL(1, 0, 1) FGEMM_INST_DECL(1, 1, 0) FGEMM_INST_DECL(1, 1, 1)
#undef FGEMM_INST_DECL

// The 8-bit kernel (K-contiguous A and B, dtype = f8_code, 256x128 tiles): one
// launch over a batch whose problems are given in 16-bit units (K, lda and ldb
// halved: the kernel moves byte pairs).
hipError_t launch_gemm_f8(const KernelKey& k, const GemmBatch& b, hipStream_t s);

int tile_m_of(int tile);
int tile_n_of(int tile);
int waves_n_of(int tile);

// Launch the classical kernel over a batch of same-shape problems.
hipError_t launch_gemm(const KernelKey& key, const GemmBatch& batch, hipStream_t stream);

// The fixed device scratch of fgemm_gemm_noalloc (noalloc.hip): its size, its
// set-up (once per device, with that device current; fgemm_create calls it) and
// its device address on a device (null before the set-up).
constexpr size_t kNoAllocScratchBytes = FGEMM_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch_init(int device);
void* noalloc_scratch(int device);

// Deterministic reduction of the per-wave partial sums of squares into ss[M].
hipError_t launch_rowsumsq_reduce(const float* partial, int parts, int M, float* ss,
                                  hipStream_t stream);

// ---------------------------------------------------------------- Strassen kernels
// A 2x2-blocked operand: base pointer, leading dimension, layout, element type and
// whether its values still need the Strassen scale.  Sub-block (bi, bj) of the
// logical (rows x cols) matrix starts at rows*bi/2, cols*bj/2.
struct BlockedOperand {
  const void* ptr;
  int64_t ld;
  int trans;          // stored transposed (logical row r, col c at ptr[c*ld + r])
  int dtype;          // ElemType in memory
  int scaled;         // 1: values already carry the scale (fp16 temporaries)
};

// max |x| of a stored rows x cols matrix as per-workgroup partial maxima (at most
// kMaxPartials of them; *count receives how many), and the power-of-two scale
// 2^floor(log2(target / max)) reduced from them.
constexpr int kMaxPartials = 4096;
hipError_t launch_maxabs(const void* X, int64_t ld, int64_t rows, int64_t cols, int dtype,
                         float* partial, int* count, hipStream_t stream);
hipError_t launch_scale_from_max(const float* partial, int count, float target, float* scale,
                                 hipStream_t stream);

// Pre-add: from the four sub-blocks of `src` (logical rows x cols), write the seven
// operands of the variant's products on that side into fp16 buffers out[0..7)
// (rows/2 x cols/2 each, same layout as src, leading dimension = their own width):
// the block sums and the plain blocks the products use, values times *scale unless
// src.scaled.  side 0 = left operand (A), 1 = right operand (B).
hipError_t launch_preadd(const BlockedOperand& src, int64_t rows, int64_t cols, int variant,
                         int side, const float* scale, void* const* out, hipStream_t stream);

// Post-add: combine seven fp32 products P[0..7) (m x n, ld = n) into the four
// blocks of the output (2m x 2n).  out32 != null: fp32 output with ld_out (plain
// combination).  Otherwise 16-bit output C (ldc) = RNE(alpha/(sa*sb) * comb
// + beta*Cin + bias).
struct PostAddArgs {
  const float* P[7];
  int64_t m, n;
  int variant;
  float* out32; int64_t ld32;
  void* C; int64_t ldc; int dtype;
  float alpha, beta;
  const void* bias;
  const float* scale_a; const float* scale_b;
  // Top level only.  rowsumsq != null: rowsumsq[r] = sum over the written row r of
  // C^2, from per-workgroup partials in ss_partial ([postadd_ss_parts(n)][2m]).
  // swiglu: op(B) had 2n columns split at the gate/up boundary, so output blocks
  // 11/21 hold gate and 12/22 up; C (2m x n) = RNE(silu(r*f*gate) * (r*f*up)
  // + beta*C) with r = 1/sqrt(rms_ss[row]*rms_inv_n + rms_eps), f = alpha/(sa*sb).
  float* rowsumsq; float* ss_partial;
  int swiglu;
  const float* rms_ss; float rms_inv_n, rms_eps;
  // act != 0 or rope_hd != 0: the activation or the rotary embedding before rounding
  int act; int rope_hd;
  const int32_t* rope_pos; int64_t rope_off; double rope_log2_base;
  // Top level only.  Bit q set: product q was formed from the unscaled inputs, so it
  // is unscaled by alpha alone (the others by alpha/(sa*sb)), in fp64.
  int unscaled;
};
hipError_t launch_postadd(const PostAddArgs& args, hipStream_t stream);
// Row-sum partials per output row the post-add writes for sub-block width n.
int64_t postadd_ss_parts(int64_t n);

// Table-driven block schemes (rectangular and tensor-decomposition LCMAs): at most
// kLinMaxBlocks blocks per operand or output and kLinMaxProducts products.
constexpr int kLinMaxBlocks = 6, kLinMaxProducts = 12;
// One pass over the br x bc logical blocks of a rows x cols operand writes the nout
// fp16 product operands out[q] = scale * sum_b coef[q*br*bc + b] * block_b (stored in
// the operand's orientation, leading dimension the stored block width).
hipError_t launch_lin_pre(const BlockedOperand& src, int64_t rows, int64_t cols, int br, int bc,
                          int nout, const signed char* coef, const float* scale, void* const* out,
                          hipStream_t stream);
// Output block (cb / nbc, cb % nbc) of C = RNE16(alpha/(sa*sb) * sum_r coef[cb*np + r] P_r
// + beta*C + bias); the products are m x n fp32 (leading dimension n).
struct LinPostArgs {
  const float* P[kLinMaxProducts];
  int np;
  int64_t m, n;
  int mbc, nbc;
  const signed char* coef;
  void* C; int64_t ldc; int dtype;
  float alpha, beta;
  const void* bias;
  const float* scale_a; const float* scale_b;
};
hipError_t launch_lin_post(const LinPostArgs& args, hipStream_t stream);

// Split-K finalize: C = RNE16(alpha * sum_s part[s] + beta*C + bias), part[s] is
// M x N fp32 (leading dimension N), C is 16-bit with leading dimension ldc.
hipError_t launch_splitk_finalize(const float* part, int splits, int64_t M, int64_t N,
                                  float alpha, float beta, void* C, int64_t ldc,
                                  const void* bias, int dtype, hipStream_t stream);

}  // namespace fgemm
