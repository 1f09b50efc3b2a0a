// Single-token decode step of the generalized gated delta rule.
//
// One token per (batch, head):  S_bar = Diag(exp(g)) S,  r = S_bar^T e,
// S = S_bar + k (z - r)^T,  o = S^T q  ("Chapter 11  Gated DeltaNet", 11.2
// and 11.3: a streaming caller hands the final state back in; the variant
// gates follow the Gated DeltaNet-2 page, key design 1, and the Q-Delta page,
// key designs 2 and 3; under the per-value-channel beta of "Chapter 11", 11.3,
// e = k and column v of the correction is scaled by beta[v]).
//
// The step is one pass over the fp32 state, so it is bound by HBM: each
// workgroup streams one head's dk x dv state in (float4 per thread, rows
// interleaved across row groups so that a row is read contiguously) and out
// again.  The two reductions over key channels (r and o) go through LDS.
#pragma once

#include "common.hpp"

namespace gdr {

struct StepParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* b;
  const float* w;
  const float* lam;
  const float* state_in;
  float* state_out;
  void* o;
  const void* gate;  // output epilogue (RMSNorm, SiLU gate), or nullptr
  const float* nw;
  float eps;
  int B, H;
  int decay, erase, write, qmix;
};

template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  constexpr int VGN = DV / 4;     // float4 column groups
  constexpr int RG = 256 / VGN;   // row groups
  constexpr int RPT = DK / RG;    // rows per thread
  static_assert(RG * VGN == 256 && RPT * RG == DK, "step layout");
  __shared__ float sA[DK], sE[DK], sK[DK], sQ[DK];
  __shared__ __attribute__((aligned(16))) float sZ[DV], sM[DV];
  __shared__ __attribute__((aligned(16))) float sR[RG][DV];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int h = bh % p.H;
  const int vgp = tid % VGN, rg = tid / VGN, v0 = vgp * 4;
  const size_t to = (size_t)bh;  // token offset: (b * 1 + 0) * H + h == bh

  // stream the state slice in first
  f32x4 S[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int c = rg + RG * m;
    S[m] = p.state_in ? *reinterpret_cast<const f32x4*>(p.state_in + ((size_t)bh * DK + c) * DV + v0)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const IO* qg = reinterpret_cast<const IO*>(p.q);
  const IO* kg = reinterpret_cast<const IO*>(p.k);
  const IO* vg = reinterpret_cast<const IO*>(p.v);
  const float beta = (p.erase == 0 || p.write == 0) ? p.beta[to] : 0.f;
  if (tid < DK) {
    const int c = tid;
    const float kv = (float)kg[to * DK + c], qv = (float)qg[to * DK + c];
    float a = 1.f;
    if (p.decay == 1) a = fexp(p.g[to]);
    else if (p.decay == 2) a = fexp(p.g[to * DK + c]);
    float e;
    if (p.erase == 1) e = p.b[to * DK + c] * kv;
    else if (p.erase == 2) e = kv;
    else e = beta * (p.qmix ? kv + (p.qmix == 2 ? p.lam[to] : p.lam[h]) * qv : kv);
    sA[c] = a;
    sE[c] = e;
    sK[c] = kv;
    sQ[c] = qv;
  }
  if (tid < DV) {
    const float vv = (float)vg[to * DV + tid];
    const float m = p.erase == 2 ? p.beta[to * DV + tid] : 1.f;
    sZ[tid] = (p.write == 1 ? p.w[to * DV + tid] : (p.erase == 2 ? m : beta)) * vv;
    sM[tid] = m;
  }
  __syncthreads();

  // forget, then predict along e: partial r over my rows
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int c = rg + RG * m;
    S[m] *= sA[c];
    r += sE[c] * S[m];
  }
  *reinterpret_cast<f32x4*>(&sR[rg][v0]) = r;
  __syncthreads();
  f32x4 rt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RG; ++j) rt += *reinterpret_cast<const f32x4*>(&sR[j][v0]);
  const f32x4 d = *reinterpret_cast<const f32x4*>(&sZ[v0]) - *reinterpret_cast<const f32x4*>(&sM[v0]) * rt;
  __syncthreads();  // sR is reused for the readout partials

  // write along k, then read along q
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int c = rg + RG * m;
    S[m] += sK[c] * d;
    o += sQ[c] * S[m];
    if (p.state_out) *reinterpret_cast<f32x4*>(p.state_out + ((size_t)bh * DK + c) * DV + v0) = S[m];
  }
  *reinterpret_cast<f32x4*>(&sR[rg][v0]) = o;
  __syncthreads();
  if (rg == 0) {
    f32x4 ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j) ot += *reinterpret_cast<const f32x4*>(&sR[j][v0]);
    if (p.gate) {
      // output epilogue ("Chapter 11", 11.3): the VGN threads of row group 0
      // hold the whole readout; RMSNorm over it, then the SiLU gate
      float ss = ot[0] * ot[0] + ot[1] * ot[1] + ot[2] * ot[2] + ot[3] * ot[3];
#pragma unroll
      for (int m = 1; m < VGN; m <<= 1) ss += __shfl_xor(ss, m, VGN);
      const float inv = rsqrtf(ss * (1.f / DV) + p.eps);
      const IO* gg = reinterpret_cast<const IO*>(p.gate) + to * DV + v0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float gv = (float)gg[u];
        ot[u] = ot[u] * inv * p.nw[v0 + u] * (gv / (1.f + fexp(-gv)));
      }
    }
    gst4(reinterpret_cast<IO*>(p.o) + to * DV + v0, ot);
  }
}

}  // namespace gdr
