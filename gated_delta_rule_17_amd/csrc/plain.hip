// Instances of the plain fp32 chunk kernel and of its two-pass form: io
// {fp32, bf16} x dk {64, 128}, value slices of 16 columns.
#include <type_traits>

#include "launch.hpp"
#include "plain_kernel.hpp"
#include "plain_split_kernel.hpp"

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

int plain_split_lds(int dk, int dvs) {
#define X(DK)                                                                    \
  if (dk == DK && dvs == 64) return plain_mrec_lds_bytes<DK>();                  \
  if (dk == DK && dvs == 16) return plain_rec_lds_bytes<DK, 16>();
  GDR_PLAIN_CASES(X)
#undef X
  return -1;
}

// the recurrence: on the matrix cores for 64-column slices, on the vector
// ALUs for 16-column ones (p.nslices follows the slice width)
template <class IO, int DK>
hipError_t plain_split_sequence(const ChunkParams& p, const BwdWs& ws, int dvs, int grid, int prep_grid,
                                hipStream_t s) {
  if (dvs == 64 && p.erase == 2) return hipErrorInvalidValue;  // the substitution needs 16-column slices
  // under a scalar decay (or none) with bf16 I/O the matrix-core recurrence
  // forms the factor rows from the inputs (half the bytes of the fp32
  // records), so the prep does not write them; with fp32 I/O the inputs
  // weigh as much as the records and the records are read
  const bool sd = dvs == 64 && p.decay != 2 && std::is_same<IO, bf16>::value;
  if (sd && p.erase == 0)
    hipLaunchKernelGGL((plain_prep_exact_kernel<DK>), dim3(prep_grid), dim3(NTHR), 0, s, p, ws);
  else
    hipLaunchKernelGGL((plain_prep_kernel<IO, DK>), dim3(prep_grid), dim3(NTHR), 0, s, p, ws, sd ? 0 : 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dvs == 64) {
    if (sd) hipLaunchKernelGGL((plain_mrec_kernel<IO, DK, false, true>), dim3(grid), dim3(2 * NTHR), 0, s, p, ws);
    else hipLaunchKernelGGL((plain_mrec_kernel<IO, DK, false, false>), dim3(grid), dim3(2 * NTHR), 0, s, p, ws);
  } else {
    hipLaunchKernelGGL((plain_rec_kernel<IO, DK, 16, false>), dim3(grid), dim3(NTHR), 0, s, p, ws);
  }
  return hipGetLastError();
}

hipError_t launch_plain_split(const ChunkParams& p, const BwdWs& ws, bool bf16io, int dk, int dvs, int grid,
                              int prep_grid, hipStream_t s) {
#define X(DK)                                                                                          \
  if (dk == DK)                                                                                        \
    return bf16io ? plain_split_sequence<bf16, DK>(p, ws, dvs, grid, prep_grid, s)                     \
                  : plain_split_sequence<float, DK>(p, ws, dvs, grid, prep_grid, s);
  GDR_PLAIN_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
