// gemm_inst.hip — instantiates the classical kernel for one (MFMA dtype, A layout,
// B layout), chosen by -DFG_DT (0 fp16, 1 bf16), -DFG_AK, -DFG_BK at compile time.
#include "gemm_mfma.h"

#ifndef FG_DT
#error "FG_DT, FG_AK and FG_BK select the instantiation"
#endif

#define FG_CAT2(a, b) a##b
#define FG_CAT(a, b) FG_CAT2(a, b)
#define FG_NAME FG_CAT(FG_CAT(FG_CAT(launch_gemm_, FG_DT), FG_CAT(_, FG_AK)), FG_BK)

namespace fgemm {

template <class CFG, int EPI, bool VEC>
static hipError_t plain(const GemmBatch& b, hipStream_t s) {
  return launch_t<CFG, FG_DT, FG_AK != 0, FG_BK != 0, EPI, VEC>(b, s);
}

template <class CFG>
static hipError_t by_epilogue(const KernelKey& k, const GemmBatch& b, hipStream_t s) {
  if (k.epi == kEpiStore16) return k.vec ? plain<CFG, kEpiStore16, true>(b, s)
                                         : plain<CFG, kEpiStore16, false>(b, s);
  // the RMS scale's share of an input gradient
  if (k.epi == kEpiRmsBwd) return k.vec ? plain<CFG, kEpiRmsBwd, true>(b, s)
                                        : plain<CFG, kEpiRmsBwd, false>(b, s);
  // an activation or the rotary embedding before the rounding
  if (k.epi == kEpiAct) return k.vec ? plain<CFG, kEpiAct, true>(b, s)
                                     : plain<CFG, kEpiAct, false>(b, s);
  if (k.epi == kEpiRope) return k.vec ? plain<CFG, kEpiRope, true>(b, s)
                                      : plain<CFG, kEpiRope, false>(b, s);
  if constexpr (CFG::FN % 2 == 0) {
    if (k.epi == kEpiSwiGLU) return k.vec ? plain<CFG, kEpiSwiGLU, true>(b, s)
                                          : plain<CFG, kEpiSwiGLU, false>(b, s);
    if (k.epi == kEpiSwiGLUBwd) return k.vec ? plain<CFG, kEpiSwiGLUBwd, true>(b, s)
                                             : plain<CFG, kEpiSwiGLUBwd, false>(b, s);
  }
  // fp32 accumulators out: Strassen sub-products and split-K partial slices
  if (k.epi == kEpiStore32 && k.vec) return plain<CFG, kEpiStore32, true>(b, s);
  return hipErrorInvalidValue;
}

hipError_t FG_NAME(const KernelKey& k, const GemmBatch& b, hipStream_t s) {
  switch (k.tile) {
    case 0: return by_epilogue<Cfg256>(k, b, s);
    case 1: return by_epilogue<Cfg128>(k, b, s);
    case 2: return by_epilogue<Cfg64>(k, b, s);
    case 3: return by_epilogue<Cfg32>(k, b, s);
    case 4: return by_epilogue<Cfg64n>(k, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fgemm
