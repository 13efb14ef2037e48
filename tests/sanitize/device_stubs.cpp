// device_stubs.cpp — link stand-ins for the library's device-side launchers, so the
// host code (argument checks, plan selection, the decision model) can be built
// alone with AddressSanitizer and UndefinedBehaviorSanitizer and run on a machine
// without a GPU.  None of these is reached by the sanitizer harness: every one
// returns an error.
#include "internal.h"

namespace fgemm {

#define FGEMM_STUB(DT, AK, BK) \
  hipError_t launch_gemm_##DT##_##AK##BK(const KernelKey&, const GemmBatch&, hipStream_t) { \
    return hipErrorNoDevice;                                                                \
  }
FGEMM_STUB(0, 0, 0) FGEMM_STUB(0, 0, 1) FGEMM_STUB(0, 1, 0) FGEMM_STUB(0, 1, 1)
FGEMM_STUB(1, 0, 0) FGEMM_STUB(1, 0, 1) FGEMM_STUB(1, 1, 0) FGEMM_STUB(1, 1, 1)
#undef FGEMM_STUB

hipError_t launch_gemm_f8(const KernelKey&, const GemmBatch&, hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_rowsumsq_reduce(const float*, int, int, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_maxabs(const void*, int64_t, int64_t, int64_t, int, float*, int* count,
                         hipStream_t) {
  *count = 0;
  return hipErrorNoDevice;
}
hipError_t launch_scale_from_max(const float*, int, float, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_preadd(const BlockedOperand&, int64_t, int64_t, int, int, const float*,
                         void* const*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_postadd(const PostAddArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lin_pre(const BlockedOperand&, int64_t, int64_t, int, int, int, const signed char*,
                          const float*, void* const*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_lin_post(const LinPostArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quantize_mx(const void*, int64_t, int64_t, int64_t, int, bool, int, void*,
                              int64_t, void*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
int64_t postadd_ss_parts(int64_t n) {  // as the post-add's grid: 256 lanes of 4 columns
  const int64_t g = (n / 4 + 255) / 256;
  return g > 0 ? g : 1;
}
hipError_t launch_splitk_finalize(const float*, int, int64_t, int64_t, float, float, void*,
                                  int64_t, const void*, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t noalloc_scratch_init(int) { return hipErrorNoDevice; }
void* noalloc_scratch(int) { return nullptr; }

}  // namespace fgemm
