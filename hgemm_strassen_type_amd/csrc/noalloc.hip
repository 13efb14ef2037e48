// noalloc.hip — the fixed device scratch behind fgemm_gemm_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) still need the classical kernel's
// scratch: the per-wave row-statistics partials and the fp32 split-K slices.  They
// live in one file-scope device array instead.  Each device the library runs on
// holds its own copy at its own address from its first fgemm_create until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is asked of the runtime once per device, with that
// device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace fgemm {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];  // device address of `scratch` per device, null until set up

}  // namespace

hipError_t noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return e != hipSuccess ? e : hipErrorInvalidSymbol;
  }
  g_addr[device] = p;
  return hipSuccess;
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_addr[device];
}

}  // namespace fgemm
