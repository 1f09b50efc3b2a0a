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
  float* T;    // [ch][64][64]  T, then dT
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
