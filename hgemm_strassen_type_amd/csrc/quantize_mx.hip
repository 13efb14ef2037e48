// quantize_mx.hip — MX quantization of 16-bit matrices for the 8-bit and 4-bit GEMMs
// (CS336 Lecture 05 notes, Page 27: a value is stored as q = cast(x/s) and used as
// s*q, with one E8M0 scale per block of 32 values; Pages 27-28: block scales make a
// transpose nontrivial, so a transposed operand is quantized on its own, its blocks
// running along the other dimension).
//
// A block's scale is 2^e with e the smallest integer such that the block's largest
// magnitude is at most the format's largest finite value times 2^e (clamped to
// [-127, 127]; 0 for an all-zero block), and each value becomes the format's nearest
// value to x / 2^e, ties to the even code, the sign kept.  x / 2^e is exact in fp32
// (a power-of-two scaling of a 16-bit value); the rounding is the hardware's
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 / v_cvt_scalef32_pk_fp4_f32 (scale 1.0), which a
// probe found bit-identical to a software round-to-nearest-even encoder (rintf of the
// value's power-of-two multiple by the format's last-bit unit, sign kept) over every
// value the quantizer can hand it: each fp16 value times 2^-24..2^8 and each bf16
// value within the format's range, 5.5 million in all.
//
// HBM-bound: 2 bytes read and 1 (8-bit) or 0.5 (4-bit) written a value, plus one
// scale byte a block.  Row-wise blocks are contiguous: four lanes share a block, each
// moving one 16-byte chunk, so every load and store instruction of a wave is one
// contiguous run.  Transposed blocks run down columns: a workgroup stages a 128 x 64
// tile in LDS as fp32 and each wave quantizes 16 of its columns, four lanes a column
// (one 32-row block each), so that the four write one output row's 128 (64) bytes.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace fgemm {
namespace {

// The largest finite value of each format as mm * 2^em, mm in [1, 2): exponent em and
// mm's fp32 mantissa bits.
template <int FMT>
struct LpFormat;
template <>
struct LpFormat<FGEMM_E4M3> {  // largest 448 = 1.75 * 2^8
  static constexpr int EM = 8;
  static constexpr uint32_t MM = 0x600000u;
};
template <>
struct LpFormat<FGEMM_E5M2> {  // largest 57344 = 1.75 * 2^15
  static constexpr int EM = 15;
  static constexpr uint32_t MM = 0x600000u;
};
template <>
struct LpFormat<FGEMM_E2M1> {  // largest 6 = 1.5 * 2^2
  static constexpr int EM = 2;
  static constexpr uint32_t MM = 0x400000u;
};

template <int DT>
__device__ __forceinline__ float load16(uint16_t h) {
  if constexpr (DT == kBF16) return __uint_as_float((uint32_t)h << 16);
  return __half2float(__ushort_as_half(h));
}

// The block exponent e for a largest magnitude amax (finite, >= 0).
template <int FMT>
__device__ __forceinline__ int block_exponent(float amax) {
  using F = LpFormat<FMT>;
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23);
  if (amax == 0.f) return 0;
  if (ef == 0) return -127;  // fp32 subnormal: far below any format's range at e = -127
  const int ea = ef - 127;
  int e = ea - F::EM + ((b & 0x7FFFFFu) > F::MM ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values v[0..3] to four codes in one dword (byte i = value i): two packed
// conversions, into the low and the high half.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float v0, float v1, float v2, float v3) {
  if constexpr (FMT == FGEMM_E4M3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  } else {
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, w, true);
  }
}

// Eight values to eight E2M1 codes in one dword (nibble i = value i).
__device__ __forceinline__ uint32_t cvt8_fp4(const float* v) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
}

// Row-wise: block blk of the matrix (row blk / bpr, block blk % bpr of that row) by
// lanes 4*blk .. 4*blk + 3 of the grid, lane c moving values 8c .. 8c+7.
template <int FMT, int DT>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ X,
                                                            int64_t ldx, int64_t rows,
                                                            int64_t bpr, uint8_t* __restrict__ Q,
                                                            int64_t ldq, uint8_t* __restrict__ S,
                                                            int64_t lds) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 2;
  const int c = (int)(gid & 3);
  const bool live = blk < rows * bpr;
  const int64_t r = live ? blk / bpr : 0, b = live ? blk % bpr : 0;
  float x[8];
  float amax = 0.f;
  if (live) {
    const uint4 raw = *reinterpret_cast<const uint4*>(X + r * ldx + 32 * b + 8 * c);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = load16<DT>((uint16_t)(w[i] & 0xFFFFu));
      x[2 * i + 1] = load16<DT>((uint16_t)(w[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }
  // the block's four lanes are adjacent: xor 1 and 2 stay inside it
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!live) return;
  const int e = block_exponent<FMT>(amax);
  if (c == 0) S[r * lds + b] = (uint8_t)(e + 127);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = ldexpf(x[i], -e);
  if constexpr (FMT == FGEMM_E2M1) {
    *reinterpret_cast<uint32_t*>(Q + r * ldq + 16 * b + 4 * c) = cvt8_fp4(x);
  } else {
    const uint32_t lo = cvt4<FMT>(x[0], x[1], x[2], x[3]);
    const uint32_t hi = cvt4<FMT>(x[4], x[5], x[6], x[7]);
    *reinterpret_cast<uint2*>(Q + r * ldq + 32 * b + 8 * c) = make_uint2(lo, hi);
  }
}

constexpr int kTR = 128, kTC = 64;  // transposed tile (fp32 in LDS, kTC words a row)

// LDS word of tile element (row, col): each 32-row band's columns rotated by 8 words,
// so that the 32 lanes of a half-wave (8 columns x 4 bands) read 32 distinct banks.
__device__ __forceinline__ int tile_at(int row, int col) {
  return row * kTC + ((col + 8 * (row >> 5)) & (kTC - 1));
}

// Transposed: the tile of source rows r0 .. r0+127, columns c0 .. c0+63 becomes rows
// c0 .. c0+63 of the quantized X^T, blocks r0/32 .. r0/32+3 of each; wave w takes
// columns c0 + 16w .., lane l column 16w + l/4 and block l%4 (source rows 32(l%4) ..).
template <int FMT, int DT>
__global__ __launch_bounds__(256) void quantize_cols_kernel(const uint16_t* __restrict__ X,
                                                            int64_t ldx, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ Q,
                                                            int64_t ldq, uint8_t* __restrict__ S,
                                                            int64_t lds) {
  __shared__ float tile[kTR * kTC];
  const int64_t r0 = (int64_t)blockIdx.y * kTR, c0 = (int64_t)blockIdx.x * kTC;
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kTR * kTC / 8 / 256; ++j) {  // 16-byte chunks, 8 a source row
    const int i = t + 256 * j;
    const int rr = i >> 3, cc = (i & 7) * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r0 + rr < rows && c0 + cc + 8 <= cols) {   // a whole chunk (ldx % 8 == 0: aligned)
      const uint4 raw = *reinterpret_cast<const uint4*>(X + (r0 + rr) * ldx + c0 + cc);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = load16<DT>((uint16_t)(w[k] & 0xFFFFu));
        v[2 * k + 1] = load16<DT>((uint16_t)(w[k] >> 16));
      }
    } else if (r0 + rr < rows && c0 + cc < cols) {  // the last columns of a row
      for (int k = 0; c0 + cc + k < cols; ++k) v[k] = load16<DT>(X[(r0 + rr) * ldx + c0 + cc + k]);
    }
    // 8 consecutive words: the rotation moves whole 8-word chunks, so none wraps
    float* dst = tile + tile_at(rr, cc);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = v[k];
  }
  __syncthreads();
  const int w = t >> 6, l = t & 63;
  const int tc = 16 * w + (l >> 2), band = l & 3;    // tile column and 32-row band
  const int64_t col = c0 + tc, rb = r0 + 32 * band;  // output row, first source row
  if (col >= cols || rb >= rows) return;            // rows % 32 == 0: a block is whole
  float x[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    x[i] = tile[tile_at(32 * band + i, tc)];
    amax = fmaxf(amax, fabsf(x[i]));
  }
  const int e = block_exponent<FMT>(amax);
  S[col * lds + rb / 32] = (uint8_t)(e + 127);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = ldexpf(x[i], -e);
  if constexpr (FMT == FGEMM_E2M1) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = cvt8_fp4(x + 8 * i);
    *reinterpret_cast<uint4*>(Q + col * ldq + rb / 2) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = cvt4<FMT>(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    uint4* dst = reinterpret_cast<uint4*>(Q + col * ldq + rb);
    dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
    dst[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
}

template <int FMT, int DT>
hipError_t launch_fmt(const void* X, int64_t rows, int64_t cols, int64_t ldx, bool transpose,
                      void* Q, int64_t ldq, void* S, int64_t lds, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint8_t* q = static_cast<uint8_t*>(Q);
  uint8_t* sc = static_cast<uint8_t*>(S);
  if (!transpose) {
    const int64_t bpr = cols / 32, lanes = rows * bpr * 4;
    const int64_t groups = (lanes + 255) / 256;
    if (groups > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_rows_kernel<FMT, DT>), dim3((unsigned)groups), dim3(256), 0, s,
                       x, ldx, rows, bpr, q, ldq, sc, lds);
  } else {
    const int64_t gx = (cols + kTC - 1) / kTC, gy = (rows + kTR - 1) / kTR;
    if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_cols_kernel<FMT, DT>), dim3((unsigned)gx, (unsigned)gy),
                       dim3(256), 0, s, x, ldx, rows, cols, q, ldq, sc, lds);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mx(const void* X, int64_t rows, int64_t cols, int64_t ldx, int dtype,
                              bool transpose, int fmt, void* Q, int64_t ldq, void* S, int64_t lds,
                              hipStream_t s) {
  if (dtype == kBF16) {
    if (fmt == FGEMM_E4M3)
      return launch_fmt<FGEMM_E4M3, kBF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
    if (fmt == FGEMM_E5M2)
      return launch_fmt<FGEMM_E5M2, kBF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
    return launch_fmt<FGEMM_E2M1, kBF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
  }
  if (fmt == FGEMM_E4M3)
    return launch_fmt<FGEMM_E4M3, kF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
  if (fmt == FGEMM_E5M2)
    return launch_fmt<FGEMM_E5M2, kF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
  return launch_fmt<FGEMM_E2M1, kF16>(X, rows, cols, ldx, transpose, Q, ldq, S, lds, s);
}

}  // namespace fgemm
