// epilogue_ops.h — elementwise transforms that an epilogue applies to the linear
// result D = alpha*acc + beta*C + bias before rounding (tilnote.io PingPong GEMM
// note: the epilogue applies elementwise operations before the store; its CODA
// section names RoPE among the operations an epilogue can take over).
//
//   activation: ReLU, SiLU x/(1+e^-x), or GELU in the tanh form of Hendrycks and
//     Gimpel, 0.5x(1 + tanh(sqrt(2/pi)(x + 0.044715x^3))), computed here as
//     x / (1 + e^(-2z)) with z the tanh argument (0.5(1 + tanh z) = 1/(1 + e^-2z));
//   RoPE: the rotary position embedding of Su et al. (RoFormer) on interleaved
//     pairs: in each head of hd columns, pair p = (2p, 2p+1) turns by
//     pos * base^(-2p/hd).  The angle is formed and reduced to [-pi, pi] in fp64
//     (at positions in the thousands an fp32 angle is off by ~1e-3 rad), then its
//     sine and cosine are taken in fp32 by the hardware instructions.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace fgemm {

__device__ __forceinline__ float apply_act(int act, float x) {
  if (act == FGEMM_ACT_RELU) return fmaxf(x, 0.f);
  if (act == FGEMM_ACT_SILU) return x / (1.f + __expf(-x));
  // GELU, tanh form
  const float z = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  return x / (1.f + __expf(-2.f * z));
}

// sin and cos of the rotation of the pair whose first column is `col` (even).
__device__ __forceinline__ void rope_sincos(int64_t pos, int col, int hd, double log2_base,
                                            float* s, float* c) {
  const int p = (col % hd) >> 1;
  const double inv_freq = exp2(-(double)(2 * p) / (double)hd * log2_base);
  const double th = (double)pos * inv_freq;
  const double two_pi = 6.283185307179586;
  const float r = (float)(th - two_pi * rint(th / two_pi));
  // hardware sine/cosine: absolute error ~1e-6 on [-pi, pi], no reduction path
  *s = __sinf(r);
  *c = __cosf(r);
}

// Transform W consecutive values of one output row starting at column col (even):
// the activation when act != 0, else the rotary embedding.
template <int W>
__device__ __forceinline__ void apply_transform(int act, const int32_t* rope_pos, int64_t rope_off,
                                                int rope_hd, double rope_log2_base, int row,
                                                int col, float (&v)[W]) {
  static_assert(W % 2 == 0, "whole pairs");
  if (act) {
#pragma unroll
    for (int e = 0; e < W; ++e) v[e] = apply_act(act, v[e]);
    return;
  }
  const int64_t pos = rope_pos ? (int64_t)rope_pos[row] : (int64_t)row + rope_off;
#pragma unroll
  for (int q = 0; q < W / 2; ++q) {
    float s, c;
    rope_sincos(pos, col + 2 * q, rope_hd, rope_log2_base, &s, &c);
    const float x0 = v[2 * q], x1 = v[2 * q + 1];
    v[2 * q] = x0 * c - x1 * s;
    v[2 * q + 1] = x0 * s + x1 * c;
  }
}

}  // namespace fgemm
