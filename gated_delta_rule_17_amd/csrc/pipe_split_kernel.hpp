// Two-pass chunkwise forward under no or a scalar decay (bf16 I/O, dk 128),
// for workloads with few heads: there the pipelined kernel of pipe_kernel.hpp
// splits each head into four or eight value slices, and every slice repeats
// the chunk's Gram tiles and inverse on its own critical path.
//
// Same chunk form as pipe_kernel.hpp ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", key design 2):
//   pass 1 (pipe_prep_kernel, one workgroup per chunk): the chunk scalars
//     (prefix sum of the log-decay, beta, beta gamma, gamma, gamma_C / gamma,
//     gamma_C), the T and A_qk tiles and A = (I + T)^{-1}, written to one
//     record per chunk in a caller-provided workspace;
//   pass 2 (pipe_fwd_kernel with PRE = true): the pipelined kernel whose
//     producer waves copy the record into LDS instead of forming it.
// Workspace record of a chunk (records ordered by (batch, head, chunk)):
//   A column-major (Acm[j][i] = A[i][j]) as a stored upper triangle | A_qk
//   row-major as a stored lower triangle (pipe_kernel.hpp: the ten non-zero
//   16 x 16 blocks of each, 320 pieces of 16 bytes) | the 336 chunk scalars
//   in the pipelined kernel's layout (PipeLay: G, beta, c_e, gamma, tail at
//   0, 64, 128, 192, 256; gamma_C at 320).
#pragma once

#include "pipe_kernel.hpp"

namespace gdr {

// Three workgroups share a CU: the k rows take the q rows' stride (this
// kernel reads both only as b128 fragments, which that stride serves without
// bank conflicts) and A takes the place of the k rows once the Gram tiles
// have read them.
template <int DK>
struct PrepPipeLay {
  using P = PipeLay<DK, 64>;  // q stride, [64][64] stride and scalar layout of the pipelined kernel
  static constexpr int SK = P::SQ, SQ = P::SQ, SC = P::SC, TDS = P::TDS, TDB = P::TDB, NSC = P::NSC;
  static constexpr int oK = 0, oQ = CH * SK * 2, oSc = oQ + CH * SQ * 2, oT = oSc + NSC * 4;
  static constexpr int oTd = oT + CH * SC * 2, TOTAL = oTd + 4 * TDB * 4;
  static constexpr int oA = oK;  // after the Gram tiles
  static_assert(CH * SC * 2 <= CH * SK * 2, "A fits in the k rows");
  static_assert(3 * TOTAL <= 160 * 1024, "three workgroups per CU");
  static_assert(oQ % 16 == 0 && oSc % 16 == 0 && oT % 16 == 0 && oTd % 16 == 0 && oA % 16 == 0, "alignment");
};

template <int DK, int GM>
__global__ __launch_bounds__(256) void pipe_prep_kernel(ChunkParams p, char* __restrict__ ws) {
  using L = PrepPipeLay<DK>;
  using R = PipeRec;
  using PL = PipeLay<DK, 64>;
  constexpr int SK = L::SK, SQ = L::SQ, SC = L::SC, TDS = L::TDS, TDB = L::TDB;
  constexpr int CG = DK / 8, TPT = CH * CG / 256;  // lane: 8 key channels x TPT tokens
  static_assert(GM == 0 || GM == 3, "the beta erase gate");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  bf16* sK = reinterpret_cast<bf16*>(smem + L::oK);
  bf16* sQ = reinterpret_cast<bf16*>(smem + L::oQ);
  float* sc = reinterpret_cast<float*>(smem + L::oSc);
  bf16* sT = reinterpret_cast<bf16*>(smem + L::oT);
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  bf16* sA = reinterpret_cast<bf16*>(smem + L::oA);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int T = p.T, H = p.H;
  const int nchunks = (T + CH - 1) / CH;
  const int job = blockIdx.x;  // (batch, head) major, chunk minor
  const int bh = job / nchunks, n = job - bh * nchunks;
  const int bb = bh / H, hh = bh - bb * H;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const float lam = p.qmix ? p.lam[hh] : 0.f;
  char* rec = ws + (size_t)job * R::BYTES;
  const int t0 = n * CH;

  // k and q rows of the chunk (zero past the end)
  {
    const bf16* kg = reinterpret_cast<const bf16*>(p.k) + seq0 * DK;
    const bf16* qg = reinterpret_cast<const bf16*>(p.q) + seq0 * DK;
    const int c0 = (tid % CG) * 8, tq0 = (tid / CG) * TPT;
    const bf16x8 zero = {};
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int t = tq0 + u;
      const size_t to = (size_t)min(t0 + t, T - 1) * H;
      const bool ok = t0 + t < T;
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kg + to * DK + c0);
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qg + to * DK + c0);
      *reinterpret_cast<bf16x8*>(sK + t * SK + c0) = ok ? kv : zero;
      *reinterpret_cast<bf16x8*>(sQ + t * SQ + c0) = ok ? qv : zero;
    }
  }
  // chunk scalars (one token per lane of wave 0)
  if (w == 0) {
    const bool ok = t0 + lane < T;
    const size_t to = (size_t)min(t0 + lane, T - 1) * H;
    const float gs = (p.decay != 0 && ok) ? p.g[seq0 + to] : 0.f;
    const float bs = p.beta[seq0 + to];
    const float G = wave_incl_scan(gs);
    const float GC = lane_value(G, 63);
    const float gam = fexp(G);
    sc[PL::sG + lane] = G;
    sc[PL::sBeta + lane] = bs;
    sc[PL::sCE + lane] = bs * gam;
    sc[PL::sGam + lane] = gam;
    sc[PL::sTail + lane] = fexp(GC - G);
    if (lane < PL::NSC - PL::sGC) sc[PL::sGC + lane] = lane == 0 ? fexp(GC) : 0.f;
  }
  __syncthreads();

  // T and A_qk tiles (the pipelined kernel's assignment); A_qk straight out
  {
    bf16* aqk_out = reinterpret_cast<bf16*>(rec + R::oAqk);
    auto tiles = [&](auto qm) __attribute__((always_inline)) {
      constexpr bool mix = decltype(qm)::value;
      const float* sG = sc + PL::sG;
      const float* sB = sc + PL::sBeta;
      switch (w) {
        case 0: scalar_gram_tiles<DK, SK, SQ, SC, TDS, TDB, mix, true>(Tiles<3, 3, 0, 3, 1, 0, 0>{}, sK, sQ, sG, sB, lam, sT,
                                                                 sTd, aqk_out, CH, g, l16); break;
        case 1: scalar_gram_tiles<DK, SK, SQ, SC, TDS, TDB, mix, true>(Tiles<3, 2, 0, 2, 1, 2, 2>{}, sK, sQ, sG, sB, lam, sT,
                                                                 sTd, aqk_out, CH, g, l16); break;
        case 2: scalar_gram_tiles<DK, SK, SQ, SC, TDS, TDB, mix, true>(Tiles<2, 1, 0, 1, 1>{}, sK, sQ, sG, sB, lam, sT, sTd,
                                                                 aqk_out, CH, g, l16); break;
        default: scalar_gram_tiles<DK, SK, SQ, SC, TDS, TDB, mix, true>(Tiles<2, 3, 2, 3, 3>{}, sK, sQ, sG, sB, lam, sT,
                                                                  sTd, aqk_out, CH, g, l16); break;
      }
    };
    if (p.qmix) tiles(IC<1>{});
    else tiles(IC<0>{});
  }
  __syncthreads();
  // A (in the k rows, read for the last time above) starts at zero, so that
  // its blocks above the diagonal stay zero
  for (int e = tid; e < CH * SC * 2 / 16; e += 256) reinterpret_cast<uint4*>(sA)[e] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  // A = (I + T)^{-1}: waves 0 and 1 split its last level
  if (w == 0) solve_inverse<SC, TDS, TDB, 1>(sTd, sT, sA, g, l16);
  else if (w == 1) solve_inverse<SC, TDS, TDB, 2>(sTd, sT, sA, g, l16);
  __syncthreads();
  for (int q = tid; q < R::PIECES_A; q += 256) {
    const TriPiece pc = tri_upper_piece(q);
    reinterpret_cast<uint4*>(rec + R::oAcm)[q] = *reinterpret_cast<const uint4*>(sA + pc.row * SC + 8 * pc.col);
  }
  if (tid < PL::NSC / 4) reinterpret_cast<uint4*>(rec + R::oSc)[tid] = reinterpret_cast<const uint4*>(sc)[tid];
}

}  // namespace gdr
