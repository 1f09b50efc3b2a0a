// Instances of the multi-token recurrent kernel (io {fp32, bf16} x dk {64,
// 128} x dv {64, 128}) and of the standalone output epilogue (dv {64, 128,
// 256}).
#include "launch.hpp"
#include "recur_kernel.hpp"

namespace gdr {

#define GDR_RECUR_CASES(X) X(128, 128) X(128, 64) X(64, 128) X(64, 64)

bool recur_supported(int dk, int dv) {
#define X(DK, DV) if (dk == DK && dv == DV) return true;
  GDR_RECUR_CASES(X)
#undef X
  return false;
}

hipError_t launch_recur(const RecurParams& p, bool bf16io, int dk, int dv, int grid, hipStream_t s) {
#define X(DK, DV)                                                                                  \
  if (dk == DK && dv == DV) {                                                                      \
    if (bf16io) hipLaunchKernelGGL((recur_fwd_kernel<bf16, DK, DV>), dim3(grid), dim3(DK * DV / 64), 0, s, p); \
    else hipLaunchKernelGGL((recur_fwd_kernel<float, DK, DV>), dim3(grid), dim3(DK * DV / 64), 0, s, p); \
    return hipGetLastError();                                                                      \
  }
  GDR_RECUR_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

bool norm_gate_supported(int dv) { return dv == 64 || dv == 128 || dv == 256; }

// rows of dv values, four waves of 64 / L rows per workgroup
hipError_t launch_norm_gate(const void* o, const void* gate, const float* nw, void* y, int64_t rows, int dv,
                            bool bf16io, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
#define X(DV)                                                                                          \
  if (dv == DV) {                                                                                      \
    if (bf16io) {                                                                                      \
      constexpr int64_t RPB = 4 * (64 / (DV / 8));                                                     \
      hipLaunchKernelGGL((norm_gate_kernel<bf16, DV>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, s,   \
                         static_cast<const bf16*>(o), static_cast<const bf16*>(gate), nw, static_cast<bf16*>(y), \
                         rows, eps);                                                                   \
    } else {                                                                                           \
      constexpr int64_t RPB = 4 * (64 / (DV / 4));                                                     \
      hipLaunchKernelGGL((norm_gate_kernel<float, DV>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, s,  \
                         static_cast<const float*>(o), static_cast<const float*>(gate), nw,             \
                         static_cast<float*>(y), rows, eps);                                           \
    }                                                                                                  \
    return hipGetLastError();                                                                          \
  }
  X(64) X(128) X(256)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
