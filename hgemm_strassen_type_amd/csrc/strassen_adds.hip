// strassen_adds.hip — the memory-bound kernels of the Strassen/Winograd path.
//
// FalconGEMM summary (euno.news), Methodology 1 and 3: a low-complexity algorithm
// replaces one product of 2x2 blocks by seven block products plus block sums, and
// kernels are grouped so shared partial results stay on chip instead of being
// fetched from DRAM again.  Here that grouping means:
//   - one pre-add kernel per operand reads its four sub-blocks once and writes the
//     seven operands of that side's products (the variant's sums and the plain
//     blocks, all as scaled fp16), chained sums (Winograd S2 from S1, S4 from S2,
//     ...) staying in registers in fp32;
//   - one post-add kernel reads the seven fp32 products once and writes all four
//     output blocks, with alpha, beta*C and the bias fused in at the top level.
// The limitation the same summary notes (temporary buffers cost memory) is why
// the temporaries are 16-bit and the products are reused level by level.
//
// Precision: sums are formed in fp32 from the exact inputs and rounded once to
// fp16.  bf16 (or large fp16) inputs are first multiplied by a power of two chosen
// from max|x| so that every sum stays inside the fp16 range; the product of the two
// scales is divided out in the final post-add.  Products accumulate in fp32.
//
// All kernels are bound by HBM bandwidth.  They stream 16-byte vectors on a 2-D
// grid: blockIdx.x walks 256 consecutive 16-byte chunks of a row (coalesced),
// blockIdx.y rows (with a stride loop when there are more rows than grid rows), so
// no lane divides an index, and every lane has several independent loads in
// flight (the four sub-blocks, the seven products, or four rows).
#include <hip/hip_runtime.h>

#include "epilogue_ops.h"
#include "internal.h"

namespace fgemm {

namespace {

// Streaming accesses: every input of these kernels is read once and every output
// written once, so their lines are non-temporal; kept in L2 they would only evict
// lines that other work reuses (Winograd/S69 depth 1 at 16384^3: 1.3-1.8 % faster in
// all).  The nontemporal builtins take native vector types, HIP's uint4 / uint2 /
// float4 are structs: these route them through.
typedef unsigned nt_v4u __attribute__((ext_vector_type(4)));
typedef unsigned nt_v2u __attribute__((ext_vector_type(2)));
typedef float nt_v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_ld(const uint4* p) {
  const nt_v4u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 nt_ld(const uint2* p) {
  const nt_v2u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v2u*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 nt_ld(const float4* p) {
  const nt_v4f v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4f*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_st(uint4 v, uint4* p) {
  __builtin_nontemporal_store(nt_v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_v4u*>(p));
}
__device__ __forceinline__ void nt_st(uint2 v, uint2* p) {
  __builtin_nontemporal_store(nt_v2u{v.x, v.y}, reinterpret_cast<nt_v2u*>(p));
}

__device__ __forceinline__ float h2f(uint32_t h, int dt) {
  return dt == kBF16 ? __uint_as_float(h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f2h16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f2h(float f, int dt) {
  return dt == kBF16 ? (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f) : f2h16(f);
}

__device__ __forceinline__ void unpack8(uint4 v, int dt, float* f) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    f[2 * p] = h2f(w[p] & 0xffffu, dt);
    f[2 * p + 1] = h2f(w[p] >> 16, dt);
  }
}
__device__ __forceinline__ uint4 pack8_f16(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) w[p] = f2h16(f[2 * p]) | (f2h16(f[2 * p + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------------ max |x|

// max |x| over a stored rows x cols matrix (leading dimension ld): every
// workgroup writes the max of its share to partial[workgroup] (no atomics; the
// scale kernel reduces the partials).  A lane reads kMaxRows rows of its chunk per
// round, independently.
constexpr int kMaxRows = 4;

__global__ void maxabs_kernel(const uint16_t* __restrict__ X, int64_t ld, int64_t rows,
                              int64_t cols, int dt, int vec, float* partial) {
  float m = 0.f;
  const int64_t chunks = (cols + 7) / 8;
  for (int64_t cx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; cx < chunks;
       cx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = cx * 8;
    const bool full = vec && c + 8 <= cols;
    for (int64_t r0 = (int64_t)blockIdx.y * kMaxRows; r0 < rows;
         r0 += (int64_t)gridDim.y * kMaxRows) {
      if (full && r0 + kMaxRows <= rows) {
        uint4 v[kMaxRows];
#pragma unroll
        for (int u = 0; u < kMaxRows; ++u)
          v[u] = nt_ld(reinterpret_cast<const uint4*>(X + (r0 + u) * ld + c));
#pragma unroll
        for (int u = 0; u < kMaxRows; ++u) {
          float f[8];
          unpack8(v[u], dt, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
        }
      } else {
        for (int64_t r = r0; r < r0 + kMaxRows && r < rows; ++r)
          for (int e = 0; e < 8 && c + e < cols; ++e) m = fmaxf(m, fabsf(h2f(X[r * ld + c + e], dt)));
      }
    }
  }
  __shared__ float wmax[4];
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    partial[blockIdx.y * gridDim.x + blockIdx.x] = b;
  }
}

// scale = 2^floor(log2(target / max)) over the partial maxima, 1 when the max is
// 0 or not finite.
__global__ void scale_from_max_kernel(const float* partial, int count, float target,
                                      float* scale) {
  float m = 0.f;
  for (int i = threadIdx.x; i < count; i += blockDim.x) m = fmaxf(m, partial[i]);
  __shared__ float wmax[4];
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x != 0) return;
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float s = 1.f;
  if (m > 0.f && isfinite(m)) {
    int e;
    // in fp64: for the smallest bf16 magnitudes target/m leaves the fp32 range
    frexp((double)target / (double)m, &e);  // target/m = f * 2^e, 0.5 <= f < 1
    e -= 1;
    e = e < -126 ? -126 : (e > 126 ? 126 : e);  // a normal fp32 power of two
    s = ldexpf(1.f, e);
  }
  *scale = s;
}

// ------------------------------------------------------------------ pre-add
// One pass over the four sub-blocks of an operand writes the seven operands of
// that side's products, in product order, as scaled fp16: the block sums (chained
// Winograd sums stay in fp32 registers) and the plain blocks, so that every
// sub-product is a plain fp16 GEMM.  A null output is skipped (a product that
// reads its plain block from the input instead).
struct PreAddArgs {
  const uint16_t* blk[4];   // X11, X12, X21, X22 (logical blocks) in storage
  int64_t ld;               // source leading dimension
  int64_t srows, scols;     // stored sub-block shape (scols contiguous)
  uint16_t* out[7];         // fp16 outputs, stored srows x scols, leading dim scols
  int dt;                   // source element type
  int scaled;               // source already carries the scale
  const float* scale;
  int variant, side;
};

__global__ void preadd_kernel(PreAddArgs a) {
  const float s = a.scaled ? 1.f : *a.scale;
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c >= a.scols) return;
  for (int64_t r = blockIdx.y; r < a.srows; r += gridDim.y) {
    int64_t si = r * a.ld + c;
    float x11[8], x12[8], x21[8], x22[8];
    unpack8(nt_ld(reinterpret_cast<const uint4*>(a.blk[0] + si)), a.dt, x11);
    unpack8(nt_ld(reinterpret_cast<const uint4*>(a.blk[1] + si)), a.dt, x12);
    unpack8(nt_ld(reinterpret_cast<const uint4*>(a.blk[2] + si)), a.dt, x21);
    unpack8(nt_ld(reinterpret_cast<const uint4*>(a.blk[3] + si)), a.dt, x22);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x11[e] *= s; x12[e] *= s; x21[e] *= s; x22[e] *= s;
    }
    const int64_t di = r * a.scols + c;
    float o[7][8];
    if (a.variant == FGEMM_VARIANT_WINOGRAD) {
      if (a.side == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float s1 = x21[e] + x22[e];   // S1 = A21 + A22
          float s2 = s1 - x11[e];       // S2 = S1 - A11
          o[0][e] = x11[e];             // P1: A11
          o[1][e] = x12[e];             // P2: A12
          o[2][e] = x12[e] - s2;        // P3: S4 = A12 - S2
          o[3][e] = x22[e];             // P4: A22
          o[4][e] = s1;                 // P5: S1
          o[5][e] = s2;                 // P6: S2
          o[6][e] = x11[e] - x21[e];    // P7: S3 = A11 - A21
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float t1 = x12[e] - x11[e];   // T1 = B12 - B11
          float t2 = x22[e] - t1;       // T2 = B22 - T1
          o[0][e] = x11[e];             // P1: B11
          o[1][e] = x21[e];             // P2: B21
          o[2][e] = x22[e];             // P3: B22
          o[3][e] = t2 - x21[e];        // P4: T4 = T2 - B21
          o[4][e] = t1;                 // P5: T1
          o[5][e] = t2;                 // P6: T2
          o[6][e] = x22[e] - x12[e];    // P7: T3 = B22 - B12
        }
      }
    } else {
      if (a.side == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[0][e] = x11[e] + x22[e];    // M1: A11 + A22
          o[1][e] = x21[e] + x22[e];    // M2: A21 + A22
          o[2][e] = x11[e];             // M3: A11
          o[3][e] = x22[e];             // M4: A22
          o[4][e] = x11[e] + x12[e];    // M5: A11 + A12
          o[5][e] = x21[e] - x11[e];    // M6: A21 - A11
          o[6][e] = x12[e] - x22[e];    // M7: A12 - A22
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[0][e] = x11[e] + x22[e];    // M1: B11 + B22
          o[1][e] = x11[e];             // M2: B11
          o[2][e] = x12[e] - x22[e];    // M3: B12 - B22
          o[3][e] = x21[e] - x11[e];    // M4: B21 - B11
          o[4][e] = x22[e];             // M5: B22
          o[5][e] = x11[e] + x12[e];    // M6: B11 + B12
          o[6][e] = x21[e] + x22[e];    // M7: B21 + B22
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 7; ++q)
      if (a.out[q]) nt_st(pack8_f16(o[q]), reinterpret_cast<uint4*>(a.out[q] + di));
  }
}

// ------------------------------------------------------------------ post-add
struct PostAddKArgs {
  const float* P[7];
  int64_t m, n;
  int variant;
  float* out32; int64_t ld32;
  uint16_t* C; int64_t ldc; int dt;
  float alpha, beta;
  const uint16_t* bias;
  const float* scale_a; const float* scale_b;
  float* ss_partial;   // [gridDim.x][2m] row-sum partials (null: no statistics)
  int swiglu;
  const float* rms_ss; float rms_inv_n, rms_eps;
  int act; int rope_hd;
  const int32_t* rope_pos; int64_t rope_off; double rope_log2_base;
  int unscaled;        // bit q: product q was formed from the unscaled inputs
};

template <class F>
__device__ __forceinline__ void combine(int variant, const F (&p)[7], F* c) {
  if (variant == FGEMM_VARIANT_WINOGRAD) {
    F u2 = p[0] + p[5];                 // U2 = P1 + P6
    F u3 = u2 + p[6];                   // U3 = U2 + P7
    F u4 = u2 + p[4];                   // U4 = U2 + P5
    c[0] = p[0] + p[1];                 // C11 = P1 + P2
    c[1] = u4 + p[2];                   // C12 = U4 + P3
    c[2] = u3 - p[3];                   // C21 = U3 - P4
    c[3] = u3 + p[4];                   // C22 = U3 + P5
  } else {
    c[0] = p[0] + p[3] - p[4] + p[6];   // C11 = M1 + M4 - M5 + M7
    c[1] = p[2] + p[4];                 // C12 = M3 + M5
    c[2] = p[1] + p[3];                 // C21 = M2 + M4
    c[3] = p[0] - p[1] + p[2] + p[5];   // C22 = M1 - M2 + M3 + M6
  }
}

// Sum of x over the workgroup's 256 lanes in a fixed order (wave64 butterfly, then
// the four waves in order); every lane gets the result.
__device__ __forceinline__ float block_sum256(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // the previous round's readers are done
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ __launch_bounds__(256) void postadd_kernel(PostAddKArgs a) {
  __shared__ float red[2][4];
  const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  // lanes past the row still take part in the row-sum reductions
  const bool active = j < a.n;
  // alpha / (sa*sb) in fp64: each scale may reach 2^126, so the factor can lie far
  // below the fp32 range while the scaled products times it are ordinary values.
  // Both scales are powers of two, so an fp32 value times the factor is exact in
  // fp64 and its one rounding is the one to fp32, as in an fp32 product.
  double factor = 1.0;
  if (!a.out32) factor = (double)a.alpha / (double)*a.scale_a / (double)*a.scale_b;
  // products of unscaled inputs carry alpha alone: every product is brought to the
  // output's scale in fp64 (exact: powers of two and fp32 values) and the seven are
  // combined there, one rounding to fp32 at the end
  const double f_unscaled = (double)a.alpha;
  const double f_out = a.unscaled ? 1.0 : factor;
  const bool stats = a.ss_partial != nullptr;
  // rotary embedding: the rates of this lane's two pairs in each column block
  // (a lane keeps its columns for every row)
  double rf[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  if (a.rope_hd && active) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int d0 = (int)((cb * a.n + j) % a.rope_hd);
      rf[cb][0] = rope_turns(d0 >> 1, a.rope_hd, a.rope_log2_base);
      rf[cb][1] = rope_turns((d0 >> 1) + 1, a.rope_hd, a.rope_log2_base);
    }
  }
  for (int64_t i = blockIdx.y; i < a.m; i += gridDim.y) {
    float ss[2] = {0.f, 0.f};  // top row i, bottom row m + i
    if (active) {
      float p[4][7];
#pragma unroll
      for (int q = 0; q < 7; ++q) {
        float4 v = nt_ld(reinterpret_cast<const float4*>(a.P[q] + i * a.n + j));
        p[0][q] = v.x; p[1][q] = v.y; p[2][q] = v.z; p[3][q] = v.w;
      }
      float c[4][4];  // [element][block]
      if (a.unscaled) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          double pd[7], cd[4];
#pragma unroll
          for (int q = 0; q < 7; ++q)
            pd[q] = ((a.unscaled >> q) & 1 ? f_unscaled : factor) * (double)p[e][q];
          combine(a.variant, pd, cd);
#pragma unroll
          for (int b = 0; b < 4; ++b) c[e][b] = (float)cd[b];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) combine(a.variant, p[e], c[e]);
      }
      if (a.swiglu) {
        // blocks 0/1 (rows i) and 2/3 (rows m + i): gate, then up
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t row = h * a.m + i;
          const double r = (double)rsqrtf(a.rms_ss[row] * a.rms_inv_n + a.rms_eps) * f_out;
          const int64_t off = row * a.ldc + j;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = (float)(r * c[e][2 * h]), u = (float)(r * c[e][2 * h + 1]);
            v[e] = g / (1.f + __expf(-g)) * u;
          }
          if (a.beta != 0.f) {
            uint2 cv = nt_ld(reinterpret_cast<const uint2*>(a.C + off));
            v[0] += a.beta * h2f(cv.x & 0xffffu, a.dt);
            v[1] += a.beta * h2f(cv.x >> 16, a.dt);
            v[2] += a.beta * h2f(cv.y & 0xffffu, a.dt);
            v[3] += a.beta * h2f(cv.y >> 16, a.dt);
          }
          nt_st(
              make_uint2(f2h(v[0], a.dt) | (f2h(v[1], a.dt) << 16),
                         f2h(v[2], a.dt) | (f2h(v[3], a.dt) << 16)), reinterpret_cast<uint2*>(a.C + off));
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t row = (b >> 1) * a.m + i, col = (b & 1) * a.n + j;
          if (a.out32) {
            *reinterpret_cast<float4*>(a.out32 + row * a.ld32 + col) =
                make_float4(c[0][b], c[1][b], c[2][b], c[3][b]);
          } else {
            const int64_t off = row * a.ldc + col;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (float)(f_out * c[e][b]);
            if (a.beta != 0.f) {
              uint2 cv = nt_ld(reinterpret_cast<const uint2*>(a.C + off));
              v[0] += a.beta * h2f(cv.x & 0xffffu, a.dt);
              v[1] += a.beta * h2f(cv.x >> 16, a.dt);
              v[2] += a.beta * h2f(cv.y & 0xffffu, a.dt);
              v[3] += a.beta * h2f(cv.y >> 16, a.dt);
            }
            if (a.bias) {
              uint2 bv = *reinterpret_cast<const uint2*>(a.bias + col);
              v[0] += h2f(bv.x & 0xffffu, a.dt);
              v[1] += h2f(bv.x >> 16, a.dt);
              v[2] += h2f(bv.y & 0xffffu, a.dt);
              v[3] += h2f(bv.y >> 16, a.dt);
            }
            if (a.act)
              apply_act_run<4>(a.act, v);
            else if (a.rope_hd)
              rope_run<4>(rope_pos_of(a.rope_pos, a.rope_off, row),
                          [&](int q) { return rf[b & 1][q]; }, v);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = f2h(v[e], a.dt);
              // statistics of the rounded, written values
              const float w = h2f(o[e], a.dt);
              ss[b >> 1] += w * w;
            }
            nt_st(make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16)), reinterpret_cast<uint2*>(a.C + off));
          }
        }
      }
    }
    if (stats) {  // uniform over the workgroup
      const float top = block_sum256(ss[0], red[0]);
      const float bot = block_sum256(ss[1], red[1]);
      if (threadIdx.x == 0) {
        float* part = a.ss_partial + (int64_t)blockIdx.x * 2 * a.m;
        part[i] = top;
        part[a.m + i] = bot;
      }
    }
  }
}

// ------------------------------------------------------------ table-driven schemes
// A block scheme given by its coefficient tables (FalconGEMM page, Methodology 1:
// tensor-decomposition LCMAs; the rectangular <2,2,3;11> among them).  One pass per
// operand side reads that side's blocks once and writes every product operand
// sum_b coef[q][b] X_b as scaled fp16; one pass over the products writes every output
// block sum_r coef[c][r] P_r with the top-level epilogue (alpha, beta*C, bias).
struct LinPreKArgs {
  const uint16_t* blk[kLinMaxBlocks];   // logical blocks in storage, block order
  int nblk;
  int64_t ld, srows, scols;             // source leading dimension, stored block shape
  uint16_t* out[kLinMaxProducts];       // fp16 outputs, stored srows x scols
  int nout;
  signed char coef[kLinMaxProducts][kLinMaxBlocks];
  int dt;
  const float* scale;
};

__global__ __launch_bounds__(256) void lin_pre_kernel(LinPreKArgs a) {
  const float s = *a.scale;
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (c >= a.scols) return;
  for (int64_t r = blockIdx.y; r < a.srows; r += gridDim.y) {
    const int64_t si = r * a.ld + c;
    float x[kLinMaxBlocks][8];
#pragma unroll
    for (int b = 0; b < kLinMaxBlocks; ++b) {
      if (b < a.nblk) {
        unpack8(nt_ld(reinterpret_cast<const uint4*>(a.blk[b] + si)), a.dt, x[b]);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[b][e] *= s;
      }
    }
    const int64_t di = r * a.scols + c;
#pragma unroll
    for (int q = 0; q < kLinMaxProducts; ++q) {
      if (q < a.nout) {
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < kLinMaxBlocks; ++b) {
          const int w = b < a.nblk ? a.coef[q][b] : 0;
          if (w != 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += (float)w * x[b][e];
          }
        }
        nt_st(pack8_f16(o), reinterpret_cast<uint4*>(a.out[q] + di));
      }
    }
  }
}

struct LinPostKArgs {
  const float* P[kLinMaxProducts];      // products, each m x n (leading dimension n)
  int np;
  int64_t m, n;
  int mbc, nbc;                         // output blocks: mbc x nbc of m x n
  signed char coef[kLinMaxBlocks][kLinMaxProducts];
  uint16_t* C; int64_t ldc; int dt;
  float alpha, beta;
  const uint16_t* bias;
  const float* scale_a; const float* scale_b;
};

__global__ __launch_bounds__(256) void lin_post_kernel(LinPostKArgs a) {
  const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (j >= a.n) return;
  // alpha / (sa*sb) in fp64, as in the Strassen post-add (both scales powers of two)
  const double factor = (double)a.alpha / (double)*a.scale_a / (double)*a.scale_b;
  for (int64_t i = blockIdx.y; i < a.m; i += gridDim.y) {
    float p[kLinMaxProducts][4];
#pragma unroll
    for (int r = 0; r < kLinMaxProducts; ++r) {
      if (r < a.np) {
        const float4 v = nt_ld(reinterpret_cast<const float4*>(a.P[r] + i * a.n + j));
        p[r][0] = v.x; p[r][1] = v.y; p[r][2] = v.z; p[r][3] = v.w;
      }
    }
#pragma unroll
    for (int cb = 0; cb < kLinMaxBlocks; ++cb) {
      if (cb < a.mbc * a.nbc) {
        float c4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kLinMaxProducts; ++r) {
          const int w = r < a.np ? a.coef[cb][r] : 0;
          if (w != 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) c4[e] += (float)w * p[r][e];
          }
        }
        const int64_t row = (int64_t)(cb / a.nbc) * a.m + i;
        const int64_t col = (int64_t)(cb % a.nbc) * a.n + j;
        const int64_t off = row * a.ldc + col;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)(factor * c4[e]);
        if (a.beta != 0.f) {
          uint2 cv = nt_ld(reinterpret_cast<const uint2*>(a.C + off));
          v[0] += a.beta * h2f(cv.x & 0xffffu, a.dt);
          v[1] += a.beta * h2f(cv.x >> 16, a.dt);
          v[2] += a.beta * h2f(cv.y & 0xffffu, a.dt);
          v[3] += a.beta * h2f(cv.y >> 16, a.dt);
        }
        if (a.bias) {
          uint2 bv = *reinterpret_cast<const uint2*>(a.bias + col);
          v[0] += h2f(bv.x & 0xffffu, a.dt);
          v[1] += h2f(bv.x >> 16, a.dt);
          v[2] += h2f(bv.y & 0xffffu, a.dt);
          v[3] += h2f(bv.y >> 16, a.dt);
        }
        nt_st(
            make_uint2(f2h(v[0], a.dt) | (f2h(v[1], a.dt) << 16),
                       f2h(v[2], a.dt) | (f2h(v[3], a.dt) << 16)), reinterpret_cast<uint2*>(a.C + off));
      }
    }
  }
}

int stream_grid(int64_t work_items) {
  // enough workgroups to cover every CU several times; grid-stride for the rest
  int64_t g = (work_items + 255) / 256;
  return (int)(g < 2048 ? (g > 0 ? g : 1) : 2048);
}

// 2-D streaming grid: 256 lanes of `per_lane`-element pieces across a row, one
// grid row per matrix row (at most 65535; the kernels loop over the rest).
dim3 rows_grid(int64_t rows, int64_t cols, int64_t per_lane) {
  int64_t gx = (cols / per_lane + 255) / 256;
  int64_t gy = rows < 65535 ? rows : 65535;
  return dim3((unsigned)(gx > 0 ? gx : 1), (unsigned)(gy > 0 ? gy : 1));
}

}  // namespace


hipError_t launch_maxabs(const void* X, int64_t ld, int64_t rows, int64_t cols, int dtype,
                         float* partial, int* count, hipStream_t stream) {
  *count = 0;
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t chunks = (cols + 7) / 8;
  int64_t gx = (chunks + 255) / 256;
  if (gx > kMaxPartials) gx = kMaxPartials;
  int64_t gy = (rows + kMaxRows - 1) / kMaxRows;
  if (gy > kMaxPartials / gx) gy = kMaxPartials / gx;
  const int vec = (ld % 8 == 0) && (reinterpret_cast<uintptr_t>(X) % 16 == 0);
  hipLaunchKernelGGL(maxabs_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(X), ld, rows, cols, dtype, vec, partial);
  *count = (int)(gx * gy);
  return hipGetLastError();
}

hipError_t launch_scale_from_max(const float* partial, int count, float target, float* scale,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_max_kernel, dim3(1), dim3(256), 0, stream, partial, count, target,
                     scale);
  return hipGetLastError();
}

hipError_t launch_preadd(const BlockedOperand& src, int64_t rows, int64_t cols, int variant,
                         int side, const float* scale, void* const* out, hipStream_t stream) {
  PreAddArgs a{};
  const uint16_t* base = static_cast<const uint16_t*>(src.ptr);
  const int64_t hr = rows / 2, hc = cols / 2;
  for (int b = 0; b < 4; ++b) {
    int bi = b >> 1, bj = b & 1;
    // logical block (bi, bj) starts at logical (bi*hr, bj*hc)
    a.blk[b] = src.trans ? base + (int64_t)bj * hc * src.ld + bi * hr
                         : base + (int64_t)bi * hr * src.ld + bj * hc;
  }
  a.ld = src.ld;
  a.srows = src.trans ? hc : hr;
  a.scols = src.trans ? hr : hc;
  for (int q = 0; q < 7; ++q) a.out[q] = static_cast<uint16_t*>(out[q]);
  a.dt = src.dtype;
  a.scaled = src.scaled;
  a.scale = scale;
  a.variant = variant;
  a.side = side;
  if (a.scols % 8 || a.ld % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(preadd_kernel, rows_grid(a.srows, a.scols, 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_postadd(const PostAddArgs& in, hipStream_t stream) {
  PostAddKArgs a{};
  for (int q = 0; q < 7; ++q) a.P[q] = in.P[q];
  a.m = in.m;
  a.n = in.n;
  a.variant = in.variant;
  a.out32 = in.out32;
  a.ld32 = in.ld32;
  a.C = static_cast<uint16_t*>(in.C);
  a.ldc = in.ldc;
  a.dt = in.dtype;
  a.alpha = in.alpha;
  a.beta = in.beta;
  a.bias = static_cast<const uint16_t*>(in.bias);
  a.scale_a = in.scale_a;
  a.scale_b = in.scale_b;
  a.swiglu = in.swiglu;
  a.rms_ss = in.rms_ss;
  a.rms_inv_n = in.rms_inv_n;
  a.rms_eps = in.rms_eps;
  a.act = in.act;
  a.rope_hd = in.rope_hd;
  a.rope_pos = in.rope_pos;
  a.rope_off = in.rope_off;
  a.rope_log2_base = in.rope_log2_base;
  a.unscaled = in.unscaled;
  if (a.unscaled && a.out32) return hipErrorInvalidValue;
  if ((a.act || a.rope_hd) && (a.out32 || !in.C || a.swiglu)) return hipErrorInvalidValue;
  if (a.n % 4) return hipErrorInvalidValue;
  const bool stats = in.rowsumsq != nullptr;
  if ((stats || a.swiglu) && (a.out32 || !in.C)) return hipErrorInvalidValue;
  if (stats && (a.swiglu || !in.ss_partial || 2 * a.m > 0x7fffffff)) return hipErrorInvalidValue;
  a.ss_partial = stats ? in.ss_partial : nullptr;
  const dim3 grid = rows_grid(a.m, a.n, 4);
  hipLaunchKernelGGL(postadd_kernel, grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && stats)
    e = launch_rowsumsq_reduce(in.ss_partial, (int)grid.x, (int)(2 * a.m), in.rowsumsq, stream);
  return e;
}

int64_t postadd_ss_parts(int64_t n) { return rows_grid(1, n, 4).x; }

hipError_t launch_lin_pre(const BlockedOperand& src, int64_t rows, int64_t cols, int br, int bc,
                          int nout, const signed char* coef, const float* scale, void* const* out,
                          hipStream_t stream) {
  const int nblk = br * bc;
  if (nblk < 1 || nblk > kLinMaxBlocks || nout < 1 || nout > kLinMaxProducts || rows % br ||
      cols % bc)
    return hipErrorInvalidValue;
  LinPreKArgs a{};
  const uint16_t* base = static_cast<const uint16_t*>(src.ptr);
  const int64_t hr = rows / br, hc = cols / bc;
  for (int b = 0; b < nblk; ++b) {
    const int bi = b / bc, bj = b % bc;
    // logical block (bi, bj) starts at logical (bi*hr, bj*hc)
    a.blk[b] = src.trans ? base + (int64_t)bj * hc * src.ld + bi * hr
                         : base + (int64_t)bi * hr * src.ld + bj * hc;
  }
  a.nblk = nblk;
  a.ld = src.ld;
  a.srows = src.trans ? hc : hr;
  a.scols = src.trans ? hr : hc;
  a.nout = nout;
  for (int q = 0; q < nout; ++q) {
    a.out[q] = static_cast<uint16_t*>(out[q]);
    for (int b = 0; b < nblk; ++b) a.coef[q][b] = coef[q * nblk + b];
  }
  a.dt = src.dtype;
  a.scale = scale;
  if (a.scols % 8 || a.ld % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lin_pre_kernel, rows_grid(a.srows, a.scols, 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_lin_post(const LinPostArgs& in, hipStream_t stream) {
  if (in.np < 1 || in.np > kLinMaxProducts || in.mbc * in.nbc < 1 ||
      in.mbc * in.nbc > kLinMaxBlocks || in.n % 4 || !in.C)
    return hipErrorInvalidValue;
  LinPostKArgs a{};
  for (int r = 0; r < in.np; ++r) a.P[r] = in.P[r];
  a.np = in.np;
  a.m = in.m;
  a.n = in.n;
  a.mbc = in.mbc;
  a.nbc = in.nbc;
  for (int cb = 0; cb < in.mbc * in.nbc; ++cb)
    for (int r = 0; r < in.np; ++r) a.coef[cb][r] = in.coef[cb * in.np + r];
  a.C = static_cast<uint16_t*>(in.C);
  a.ldc = in.ldc;
  a.dt = in.dtype;
  a.alpha = in.alpha;
  a.beta = in.beta;
  a.bias = static_cast<const uint16_t*>(in.bias);
  a.scale_a = in.scale_a;
  a.scale_b = in.scale_b;
  hipLaunchKernelGGL(lin_post_kernel, rows_grid(a.m, a.n, 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ split-K finalize
namespace {
// Sums the fp32 K slices of a skinny GEMM in a fixed order and applies the
// epilogue; four consecutive columns per lane where the row allows it.
__global__ void splitk_finalize_kernel(const float* __restrict__ part, int splits, int64_t M,
                                       int64_t N, float alpha, float beta, uint16_t* C,
                                       int64_t ldc, const uint16_t* bias, int dt) {
  const int64_t chunks = (N + 3) / 4;
  const int64_t total = M * chunks;
  const int64_t slice = M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / chunks, j = (t - i * chunks) * 4;
    const int nv = N - j < 4 ? (int)(N - j) : 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sidx = 0; sidx < splits; ++sidx) {
      const float* p = part + sidx * slice + i * N + j;
      if (nv == 4 && (N & 3) == 0) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
      } else {
        for (int e = 0; e < nv; ++e) v[e] += p[e];
      }
    }
    uint16_t* c = C + i * ldc + j;
    for (int e = 0; e < nv; ++e) {
      float r = alpha * v[e];
      if (beta != 0.f) r += beta * h2f(c[e], dt);
      if (bias) r += h2f(bias[j + e], dt);
      c[e] = (uint16_t)f2h(r, dt);
    }
  }
}
}  // namespace

hipError_t launch_splitk_finalize(const float* part, int splits, int64_t M, int64_t N,
                                  float alpha, float beta, void* C, int64_t ldc,
                                  const void* bias, int dtype, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_finalize_kernel, dim3(stream_grid(M * ((N + 3) / 4))), dim3(256), 0,
                     stream, part, splits, M, N, alpha, beta, static_cast<uint16_t*>(C), ldc,
                     static_cast<const uint16_t*>(bias), dtype);
  return hipGetLastError();
}

// ------------------------------------------------------------ row sum reduction
namespace {
__global__ void rowsumsq_reduce_kernel(const float* __restrict__ part, int parts, int M,
                                       float* __restrict__ ss) {
  int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= M) return;
  float s = 0.f;
  for (int p = 0; p < parts; ++p) s += part[(int64_t)p * M + row];
  ss[row] = s;
}
}  // namespace

hipError_t launch_rowsumsq_reduce(const float* partial, int parts, int M, float* ss,
                                  hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(rowsumsq_reduce_kernel, dim3((M + 255) / 256), dim3(256), 0, stream, partial,
                     parts, M, ss);
  return hipGetLastError();
}

}  // namespace fgemm
