// fp32 I/O with fp32 MFMA (v_mfma_f32_16x16x4_f32) throughout, for the
// tighter fp32 tolerance.  dk = 64 only: at dk = 128 the fp32 operand tiles
// do not fit the 160 KB of LDS.
#include "launch.hpp"

namespace gdr {

#define GDR_F32_CASES(X) \
  X(64, 32, false) X(64, 16, false) X(64, 32, true) X(64, 16, true)

int chunk_lds_f32(int dk, int dvs, bool chan) {
#define X(DK, DVS, CHAN) \
  if (dk == DK && dvs == DVS && chan == CHAN) return chunk_lds_bytes<float, DK, DVS, CHAN>();
  GDR_F32_CASES(X)
#undef X
  return -1;
}

hipError_t launch_chunk_f32(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s) {
#define X(DK, DVS, CHAN)                                                                    \
  if (dk == DK && dvs == DVS && chan == CHAN) {                                             \
    hipLaunchKernelGGL((chunk_fwd_kernel<float, float, DK, DVS, CHAN>), dim3(grid), dim3(NTHR), 0, s, p); \
    return hipGetLastError();                                                               \
  }
  GDR_F32_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
