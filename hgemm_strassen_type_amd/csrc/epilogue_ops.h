// epilogue_ops.h — elementwise transforms that an epilogue applies to the linear
// result D = alpha*acc + beta*C + bias before rounding (tilnote.io PingPong GEMM
// note: the epilogue applies elementwise operations before the store; its CODA
// section names RoPE among the operations an epilogue can take over).
//
//   activation: ReLU, SiLU x/(1+e^-x), or GELU in the tanh form of Hendrycks and
//     Gimpel, 0.5x(1 + tanh(sqrt(2/pi)(x + 0.044715x^3))), computed here as
//     x / (1 + e^(-2z)) with z the tanh argument (0.5(1 + tanh z) = 1/(1 + e^-2z));
//     1.5957691216057308 below is 2*sqrt(2/pi);
//   RoPE: the rotary position embedding of Su et al. (RoFormer) on interleaved
//     pairs: in each head of hd columns, pair p = (2p, 2p+1) turns by
//     pos * base^(-2p/hd).  The pair rates base^(-2p/hd)/(2 pi) are computed once
//     in fp64; the angle is formed in turns and reduced in fp64 (at positions in
//     the thousands an fp32 angle is off by ~1e-3 rad), and its sine and cosine
//     are taken in fp32 by the hardware instructions.  The GPU path needs hd to be a
//     multiple of 8, so the 4 or 8 consecutive columns a lane transforms never
//     leave their head.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace fgemm {

constexpr int kRopeMaxPairs = 512;  // head widths up to 1024

// SiLU and GELU are both x * sigmoid(t), with t = x or t = 2z; one exponential and
// one hardware reciprocal (1 ulp) per value keep the unrolled epilogue small.
__device__ __forceinline__ float apply_act(int act, float x) {
  const float t = act == FGEMM_ACT_GELU_TANH ? 1.5957691216057308f * (x + 0.044715f * x * x * x)
                                             : x;
  const float y = x * __builtin_amdgcn_rcpf(1.f + __expf(-t));
  return act == FGEMM_ACT_RELU ? fmaxf(x, 0.f) : y;
}

template <int W>
__device__ __forceinline__ void apply_act_run(int act, float (&v)[W]) {
#pragma unroll
  for (int e = 0; e < W; ++e) v[e] = apply_act(act, v[e]);
}

// Rotation rate of pair p of a head of hd columns in turns per position:
// base^(-2p/hd) / (2 pi).
__device__ __forceinline__ double rope_turns(int p, int hd, double log2_base) {
  const double inv_two_pi = 0.15915494309189535;
  return exp2(-(double)(2 * p) / (double)hd * log2_base) * inv_two_pi;
}

// Rotate the pairs of W consecutive values at position `pos`; turns(q) is the
// rotation rate of pair q of the run.  The angle in turns is reduced to
// [-1/2, 1/2] in fp64 and handed to the hardware sine and cosine, which take
// their argument in turns (absolute error ~1e-6).
template <int W, class F>
__device__ __forceinline__ void rope_run(double pos, const F& turns, float (&v)[W]) {
  static_assert(W % 2 == 0, "whole pairs");
#pragma unroll
  for (int q = 0; q < W / 2; ++q) {
    const double t = pos * turns(q);
    const float r = (float)(t - rint(t));
    const float s = __builtin_amdgcn_sinf(r), c = __builtin_amdgcn_cosf(r);
    const float x0 = v[2 * q], x1 = v[2 * q + 1];
    v[2 * q] = x0 * c - x1 * s;
    v[2 * q + 1] = x0 * s + x1 * c;
  }
}

// Position of output row `row` for the rotary embedding.
__device__ __forceinline__ double rope_pos_of(const int32_t* pos, int64_t off, int64_t row) {
  return pos ? (double)pos[row] : (double)(row + off);
}

}  // namespace fgemm
