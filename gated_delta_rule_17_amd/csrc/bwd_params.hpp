// Parameter structs of the backward (bwd_kernel.hpp), shared by the kernel
// translation units and the host code.
#pragma once

#include "chunk_kernel.hpp"

namespace gdr {

// Workspace arrays of the backward, fp32, indexed by chunk-head
// ch = (batch * H + head) * n_chunks + chunk.
struct BwdWs {
  float* S;    // [ch][DK][DV]  state entering the chunk
  float* W;    // [ch][64][DV]  W = A (Z - E_bar S)
  float* dR;   // [ch][64][DV]  dR = A^T dW (= dZ)
  float* dS;   // [ch][DK][DV]  gradient of the state leaving the chunk
  float* T;    // [ch][64][64]  A = (I + T)^{-1} (T under the per-value-channel beta), then dT
  float* A;    // [ch][64][64]  A_qk, then dA_qk
  float* Eb;   // [ch][64][DK]  E_bar, then dE_bar
  float* Qg;   // [ch][64][DK]  Q_gamma, then dQ_gamma
  float* Kt;   // [ch][64][DK]  K_tail, then dK_tail
  float* gC;   // [ch][DK]      gamma_C, then sum_v S dS
  float* dlam; // [B,T,H]       per-token lambda gradients (a per-head lambda sums them)
};

struct BwdParams {
  ChunkParams f;      // the forward's inputs and kinds (o, state_out unused)
  const void* d_o;    // [B,T,H,dv] io dtype
  const float* d_st;  // [B,H,dk,dv] or nullptr (zero)
  float *dq, *dk, *dv, *dg, *dbeta, *db, *dw, *dlam, *dstate;
  BwdWs ws;
  int nchunks;
};

}  // namespace gdr

namespace gdr {

// Record arrays of the two-pass plain form (plain_split_kernel.hpp) in one
// workspace, fp32, each array 256-byte aligned, nrec = B * H * n_chunks
// records: T, Aqk [nrec][64][64]; E_bar, Q_gamma, K_tail [nrec][64][dk];
// gamma_C [nrec][dk].  The other arrays of the returned BwdWs are null.
inline int64_t plain_split_layout(int64_t nrec, int dk, char* base, BwdWs* out) {
  int64_t off = 0;
  auto take = [&](int64_t floats) {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += (floats * 4 + 255) / 256 * 256;
    return p;
  };
  BwdWs w{};
  w.T = take(nrec * CH * CH);
  w.A = take(nrec * CH * CH);
  w.Eb = take(nrec * CH * dk);
  w.Qg = take(nrec * CH * dk);
  w.Kt = take(nrec * CH * dk);
  w.gC = take(nrec * dk);
  if (out) *out = w;
  return off;
}

}  // namespace gdr
