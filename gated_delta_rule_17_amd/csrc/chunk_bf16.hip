// bf16 I/O, bf16 MFMA operands, fp32 accumulation and fp32 state.
#include "launch.hpp"

namespace gdr {

#define GDR_BF16_CASES(X) \
  X(128, 64, false) X(128, 32, false) X(128, 16, false) \
  X(128, 64, true)  X(128, 32, true)  X(128, 16, true)  \
  X(64, 64, false)  X(64, 32, false)  X(64, 16, false)  \
  X(64, 64, true)   X(64, 32, true)   X(64, 16, true)

int chunk_lds_bf16(int dk, int dvs, bool chan) {
#define X(DK, DVS, CHAN) \
  if (dk == DK && dvs == DVS && chan == CHAN) return chunk_lds_bytes<bf16, DK, DVS, CHAN>();
  GDR_BF16_CASES(X)
#undef X
  return -1;
}

hipError_t launch_chunk_bf16(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s) {
#define X(DK, DVS, CHAN)                                                                  \
  if (dk == DK && dvs == DVS && chan == CHAN) {                                           \
    hipLaunchKernelGGL((chunk_fwd_kernel<bf16, bf16, DK, DVS, CHAN>), dim3(grid), dim3(NTHR), 0, s, p); \
    return hipGetLastError();                                                             \
  }
  GDR_BF16_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
