// Instances and launch sequence of the backward (bwd_kernel.hpp): io {fp32,
// bf16} x dk {64, 128} x dv {64, 128}.
#include <type_traits>

#include "bwd_kernel.hpp"
#include "launch.hpp"
#include "plain_split_kernel.hpp"

namespace gdr {

#define GDR_BWD_CASES(X) X(128, 128) X(128, 64) X(64, 128) X(64, 64)

bool bwd_supported(int dk, int dv) {
#define X(DK, DV) if (dk == DK && dv == DV) return true;
  GDR_BWD_CASES(X)
#undef X
  return false;
}

template <class IO, int DK, int DV>
hipError_t bwd_sequence(const BwdParams& p, int BH, hipStream_t s) {
  const int N = p.nchunks;
  // record pass: the chunk records once per chunk, then the recurrence of
  // each slice writing its entering states and W
  // (the recurrence on the matrix cores, slices of 64 columns; the backward
  // takes no per-value-channel beta)
  // under a scalar decay (or none) with bf16 I/O the recurrence and the
  // state pass form E_bar, Q_gamma, K_tail and gamma_C from the inputs (half
  // the bytes of the fp32 records): the prep does not write them
  const bool sd = p.f.decay != 2 && std::is_same<IO, bf16>::value;
  if (N > 0) {
    if (sd && p.f.erase == 0)
      hipLaunchKernelGGL((plain_prep_exact_kernel<DK>), dim3(BH * N), dim3(NTHR), 0, s, p.f, p.ws);
    else
      hipLaunchKernelGGL((plain_prep_kernel<IO, DK>), dim3(BH * N), dim3(NTHR), 0, s, p.f, p.ws, sd ? 0 : 1);
    ChunkParams f64 = p.f;
    f64.nslices = DV / 64;
    if (sd)
      hipLaunchKernelGGL((plain_mrec_kernel<IO, DK, true, true>), dim3(BH * f64.nslices), dim3(2 * NTHR), 0, s, f64,
                         p.ws);
    else
      hipLaunchKernelGGL((plain_mrec_kernel<IO, DK, true, false>), dim3(BH * f64.nslices), dim3(2 * NTHR), 0, s, f64,
                         p.ws);
  }
  if (sd) hipLaunchKernelGGL((bwd_state_mfma_kernel<IO, DK, true>), dim3(BH * (DV / 64)), dim3(2 * NTHR), 0, s, p);
  else hipLaunchKernelGGL((bwd_state_mfma_kernel<IO, DK, false>), dim3(BH * (DV / 64)), dim3(2 * NTHR), 0, s, p);
  if (N > 0) {
    // the products over the value channels, then the key pass: per term
    // under a decay per key channel; under a scalar decay (or none) both in
    // one kernel, on the matrix cores
    if (p.f.decay == 2) {
      hipLaunchKernelGGL((bwd_prod_kernel<IO, DK, DV>), dim3(BH * N), dim3(NTHR), 0, s, p);
      hipLaunchKernelGGL((bwd_key_kernel<IO, DK, DV>), dim3(BH * N), dim3(NTHR), 0, s, p);
    } else {
      hipLaunchKernelGGL((bwd_prodkey_kernel<IO, DK, DV>), dim3(BH * N), dim3(NTHR), 0, s, p);
    }
  }
  if (p.f.qmix == 1)
    hipLaunchKernelGGL(bwd_lam_reduce_kernel, dim3(p.f.H), dim3(256), 0, s, p.ws.dlam, p.dlam, p.f.B, p.f.T, p.f.H);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, bool bf16io, int dk, int dv, int BH, hipStream_t s) {
#define X(DK, DV)                                                             \
  if (dk == DK && dv == DV)                                                   \
    return bf16io ? bwd_sequence<bf16, DK, DV>(p, BH, s) : bwd_sequence<float, DK, DV>(p, BH, s);
  GDR_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdr
