// Instances of the plain fp32 chunk kernel: io {fp32, bf16} x dk {64, 128},
// value slices of 16 columns.
#include "launch.hpp"
#include "plain_kernel.hpp"

namespace gdr {

#define GDR_PLAIN_CASES(X) X(64) X(128)

int plain_lds(int dk) {
#define X(DK) if (dk == DK) return plain_lds_bytes<DK, 16>();
  GDR_PLAIN_CASES(X)
#undef X
  return -1;
}

hipError_t launch_plain(const ChunkParams& p, bool bf16io, int dk, int grid, hipStream_t s) {
#define X(DK)                                                                                   \
  if (dk == DK) {                                                                               \
    if (bf16io) hipLaunchKernelGGL((plain_fwd_kernel<bf16, DK, 16>), dim3(grid), dim3(NTHR), 0, s, p, BwdWs{}); \
    else hipLaunchKernelGGL((plain_fwd_kernel<float, DK, 16>), dim3(grid), dim3(NTHR), 0, s, p, BwdWs{});   \
    return hipGetLastError();                                                                   \
  }
  GDR_PLAIN_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
