// gemm_f8.hip — instantiates the GEMM kernel for 8-bit inputs (CS336 Lecture 05
// notes, Page 27: FP8 E4M3 and E5M2), both operands K-contiguous, for every pair of
// input formats, per-tensor or MX block scales, and both 16-bit output types, with
// the 16-bit store epilogue; and for 4-bit E2M1 inputs with MX block scales (Page
// 29 of the same notes).
#include "gemm_mfma.h"

namespace fgemm {

template <int FA, int FB, int MX>
static hipError_t by_output(const KernelKey& k, const GemmBatch& b, hipStream_t s) {
  constexpr int DT = f8_code(FA, FB, MX);
  if (k.odt == kBF16) return launch_t<CfgF8, DT, true, true, kEpiStore16, true, kBF16>(b, s);
  if (k.odt == kF16) return launch_t<CfgF8, DT, true, true, kEpiStore16, true, kF16>(b, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f8(const KernelKey& k, const GemmBatch& b, hipStream_t s) {
  if (!k.a_kcontig || !k.b_kcontig || !k.vec || k.epi != kEpiStore16) return hipErrorInvalidValue;
  switch (k.dtype) {
    case f8_code(0, 0): return by_output<0, 0, 0>(k, b, s);
    case f8_code(0, 1): return by_output<0, 1, 0>(k, b, s);
    case f8_code(1, 0): return by_output<1, 0, 0>(k, b, s);
    case f8_code(1, 1): return by_output<1, 1, 0>(k, b, s);
    // MXFP8: E8M0 scales per block of 32 (Page 27 of the same notes)
    case f8_code(0, 0, 1): return by_output<0, 0, 1>(k, b, s);
    case f8_code(0, 1, 1): return by_output<0, 1, 1>(k, b, s);
    case f8_code(1, 0, 1): return by_output<1, 0, 1>(k, b, s);
    case f8_code(1, 1, 1): return by_output<1, 1, 1>(k, b, s);
    // MXFP4: E2M1 values, E8M0 scales per block of 32
    case kF4MX:
      if (k.odt == kBF16) return launch_t<CfgF4, kF4MX, true, true, kEpiStore16, true, kBF16>(b, s);
      if (k.odt == kF16) return launch_t<CfgF4, kF4MX, true, true, kEpiStore16, true, kF16>(b, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace fgemm
