// Decode-step kernel instances.
#include "launch.hpp"

namespace gdr {

#define GDR_STEP_CASES(X) X(128, 128) X(128, 64) X(64, 128) X(64, 64)

bool step_supported(int dk, int dv) {
#define X(DK, DV) if (dk == DK && dv == DV) return true;
  GDR_STEP_CASES(X)
#undef X
  return false;
}

hipError_t launch_step(const StepParams& p, int io_bf16, int dk, int dv, int grid, hipStream_t s) {
#define X(DK, DV)                                                                            \
  if (dk == DK && dv == DV) {                                                                \
    if (io_bf16) hipLaunchKernelGGL((step_kernel<bf16, DK, DV>), dim3(grid), dim3(256), 0, s, p); \
    else hipLaunchKernelGGL((step_kernel<float, DK, DV>), dim3(grid), dim3(256), 0, s, p);    \
    return hipGetLastError();                                                                \
  }
  GDR_STEP_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
