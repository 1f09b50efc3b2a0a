// Pipelined chunkwise forward of the generalized gated delta rule on gfx950
// for bf16 inputs with a per-key-channel decay (KDA, Gated DeltaNet-2): erase
// gate beta or per key channel (b), write gate beta or per value channel (w),
// and the Q-Delta mix with the beta erase gate.
//
// Same chunk form as pipe_kernel.hpp ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", key design 2, with W = A (Z - E_bar S)); with a
// decay per key channel the scalings cannot move to accumulator rows, so the
// operands are formed explicitly:
//   E_bar = e * gamma,  Q_gamma = q * gamma,  K_tail = k * gamma_C / gamma
//   (elementwise, per token and key channel; all <= |input|)
// and the Gram entries T[i][j] = sum_c e_i[c] k_j[c] exp(G_i[c] - G_j[c]) are
// formed from bounded factors around the first token s_J = 16 J of each
// 16-token block J (gamma^{-1} is never formed):
//   xe_i = e_i exp(G_i - G_{s_I}) <= 1,   xq_i = q_i exp(G_i - G_{s_I}) <= 1
//   kb_j = k_j exp(G_{s_J} - G_j)  in [1, exp(window)]
//   tile (I, J < I):  T = xe_I diag(d_IJ) kb_J^T,  d_IJ = exp(G_{s_I} - G_{s_J}) <= 1
//   tile (I, I):      T = xe_I kb_I^T, entries above the diagonal masked
// The window of a block (largest decay of a channel across it) bounds kb; a
// chunk with a window above WINDOW_LIMIT computes its tiles exactly in fp32
// instead (see gram_exact).
//
// Workgroup: the consumer waves of pipe_kernel.hpp, four elementwise waves
// (wave w owns the 16-token block w: log-decay prefix sums, bounded factors,
// E_bar, Q_gamma, K_tail, its diagonal Gram tile) and two Gram waves (the six
// tiles below the diagonal blocks; wave 0 inverts I + T, wave 1 forms the
// per-(block, channel) constants of the next chunk).  One chunk step = three
// barriers.  The per-chunk operands do not fit twice in LDS, so each has one
// buffer, written in the phase after its last reader:
//   region   written by producers      read by consumers
//   E        phase 3 (E_bar, Q_gamma)  phase 1 (K S, Q S)
//   P        phase 1 (kb, xe, xq)      -           (producer Gram, phase 2;
//                                                   consumer O staging, phase 3)
//   C        phase 3 (Z, A, A_qk)      phase 2 (W, O)
//   K        phase 1 of the next step  phase 3 (state update)
//            (K_tail)
// Region E is free in phase 2 and holds the exact-Gram staging when needed.
// Inside the step loops every prefetch is unconditional (indices clamped to
// the last chunk): registers written under a condition that the compiler
// cannot tie to their use stay live across the whole loop.
#pragma once

#include "chunk_kernel.hpp"
#include "pipe_kernel.hpp"

namespace gdr {

// A list of (I, J) 16x16 tiles of T and A_qk: TileList<I0, J0, I1, J1, ...>
template <int... P>
struct TileList {
  static constexpr int n = sizeof...(P) / 2;
  static constexpr int v[sizeof...(P)] = {P...};
  static constexpr int I(int t) { return v[2 * t]; }
  static constexpr int J(int t) { return v[2 * t + 1]; }
};

// ---- T and A_qk tiles of one chunk, shared by the kernels of this file and
// chan_split_kernel.hpp ------------------------------------------------------
// Both kinds per tile, computed transposed (D^T = kb_J X_I^T), so that each
// lane holds four consecutive columns j of one row i (lane l: row 16 I + l %
// 16, columns 16 J + 4 (l / 16) + r).

// Bounded-factor products: kb, xe, xq rows of stride SE, d_IJ rows of DK.
template <int DK, int SE, class TL>
__device__ __forceinline__ void gram_bounded_tiles(TL, const bf16* sKb, const bf16* sXe, const bf16* sXq,
                                                   const float* sD, f32x4* accT, f32x4* accA, int g, int l16) {
  constexpr int NKS = DK / 32;
#pragma unroll
  for (int t = 0; t < TL::n; ++t) {
    const int I = TL::I(t), J = TL::J(t);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      bf16x8 kj = *reinterpret_cast<const bf16x8*>(sKb + (16 * J + l16) * SE + 32 * s + 8 * g);
      if (J < I) {
        const float* d = sD + (I * (I - 1) / 2 + J) * DK + 32 * s + 8 * g;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(d), d1 = *reinterpret_cast<const f32x4*>(d + 4);
        f32x4 lo = {(float)kj[0], (float)kj[1], (float)kj[2], (float)kj[3]};
        f32x4 hi = {(float)kj[4], (float)kj[5], (float)kj[6], (float)kj[7]};
        kj = cat8(cvt4(lo * d0), cvt4(hi * d1));
      }
      const bf16x8 xe = *reinterpret_cast<const bf16x8*>(sXe + (16 * I + l16) * SE + 32 * s + 8 * g);
      const bf16x8 xq = *reinterpret_cast<const bf16x8*>(sXq + (16 * I + l16) * SE + 32 * s + 8 * g);
      accT[t] = mma32(kj, xe, accT[t]);
      accA[t] = mma32(kj, xq, accA[t]);
    }
  }
}

// Exact entries sum_c x_i[c] k_j[c] exp(G_i[c] - G_j[c]) in fp32, for chunks
// whose block windows exceed the limit: over slabs of SW channels staged by
// this wave alone in st ([64 tokens][4][SW] floats; one token per lane).
// The log-decay cumsum here is in natural units.
template <int DK, int SW, bool ERASE_CH, class TL>
__device__ __forceinline__ void gram_exact_tiles(TL, float* st, const bf16* kg, const bf16* qg, const float* g_seq,
                                                 const float* b_seq, const float* beta_seq, bool qmix, float lam,
                                                 int n, int T, int H, f32x4* accT, f32x4* accA, int lane, int g,
                                                 int l16) {
  const int t0 = n * CH;
  const int t = lane;
  const bool ok = t0 + t < T;
  const int to = min(t0 + t, T - 1) * H;
#pragma unroll 1
  for (int cs = 0; cs < DK; cs += SW) {
#pragma unroll 1
    for (int c = 0; c < SW; ++c) {
      const int a = to * DK + cs + c;
      const float kv = ok ? (float)kg[a] : 0.f;
      const float qv = ok ? (float)qg[a] : 0.f;
      float ev;
      if constexpr (ERASE_CH) ev = (ok ? b_seq[a] : 0.f) * kv;
      else ev = (ok ? beta_seq[to] : 0.f) * (qmix ? kv + lam * qv : kv);
      st[t * 4 * SW + c] = wave_incl_scan(ok ? g_seq[a] : 0.f);
      st[t * 4 * SW + SW + c] = ev;
      st[t * 4 * SW + 2 * SW + c] = kv;
      st[t * 4 * SW + 3 * SW + c] = qv;
    }
    // (one wave: its staging writes complete before these reads)
#pragma unroll 1
    for (int c = 0; c < SW; ++c) {
#pragma unroll
      for (int tt = 0; tt < TL::n; ++tt) {
        const int i = 16 * TL::I(tt) + l16, j0 = 16 * TL::J(tt) + 4 * g;
        const float Gi = st[i * 4 * SW + c], ei = st[i * 4 * SW + SW + c], qi = st[i * 4 * SW + 3 * SW + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          const float Gj = st[j * 4 * SW + c], kj = st[j * 4 * SW + 2 * SW + c];
          const float ex = (j <= i) ? fexp(Gi - Gj) : 0.f;
          accT[tt][r] += ei * kj * ex;
          accA[tt][r] += qi * kj * ex;
        }
      }
    }
  }
}

// Masks (T: j < i, A_qk: j <= i); T below the diagonal blocks to bf16 rows
// of stride SC, its diagonal blocks to fp32 rows (block stride TDB, row
// stride TDS); A_qk returned in aqk.
template <int SC, int TDS, int TDB, class TL>
__device__ __forceinline__ void gram_mask_tiles(TL, const f32x4* accT, const f32x4* accA, f32x4* aqk, bf16* sT,
                                                float* sTd, int g, int l16) {
#pragma unroll
  for (int t = 0; t < TL::n; ++t) {
    const int I = TL::I(t), J = TL::J(t);
    const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
    f32x4 xT, xA;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      xT[r] = (j0 + r < i) ? accT[t][r] : 0.f;
      xA[r] = (j0 + r <= i) ? accA[t][r] : 0.f;
    }
    aqk[t] = xA;
    if (J < I) *reinterpret_cast<bf16x4*>(sT + i * SC + j0) = cvt4(xT);
    else *reinterpret_cast<f32x4*>(sTd + I * TDB + l16 * TDS + 4 * g) = xT;
  }
}

template <int DK, int DVS>
struct ChanLay {
  static constexpr int SE = DK + 8;                       // rows of E_bar, Q_gamma, kb, xe, xq
  static constexpr int SKT = DK + (DK == 128 ? 32 : 24);  // K_tail rows (transposing reads)
  static constexpr int SC = CH + 8, SZ = DVS + 8, SO = CH + 8;
  static constexpr int TDS = 20, TDB = 16 * TDS;
  static constexpr int SW = DK / 32;  // channels per slab of the exact Gram
  static constexpr int szE = CH * SE * 2;
  static constexpr int oEb = 0, oQg = oEb + szE;                            // region E
  static constexpr int oKb = oQg + szE, oXe = oKb + szE, oXq = oXe + szE;  // region P
  static constexpr int oZ = oXq + szE;                                     // region C
  static constexpr int oAcm = oZ + CH * SZ * 2;
  static constexpr int oAqk = oAcm + CH * SC * 2;
  static constexpr int oKt = oAqk + CH * SC * 2;  // region K
  // per-(block, key channel) constants of a chunk, rows of DK floats:
  //   0-3   exp(G_sJ), even chunks          E_bar = xe * row, Q_gamma = xq * row
  //   4-7   exp(G_C - G_sJ)                 K_tail = kb * row
  //   8-13  d_IJ = exp(G_sI - G_sJ), row 8 + I (I - 1) / 2 + J
  //   14-15 gamma_C = exp(G_C), by chunk parity
  //   16-19 exp(G_sJ), odd chunks
  static constexpr int oCst = oKt + CH * SKT * 2;
  // in-block prefix sums of the log-decay of the next chunk, rows of DK
  // floats: 0-3 at the first token of block J, 4-7 at its last token
  static constexpr int oBt = oCst + 20 * DK * 4;
  static constexpr int oT = oBt + 8 * DK * 4;     // T below the diagonal, bf16 rows
  // diagonal blocks of T, fp32 rows of TDS floats (columns 16-19 unused: row
  // 0 holds the two exact-Gram flags, by chunk parity, in columns 16-17)
  static constexpr int oTd = oT + CH * SC * 2;
  static constexpr int TOTAL = oTd + 4 * TDB * 4;
  static_assert(6 * CH * 4 * SW * 4 <= 2 * szE, "exact-Gram staging does not fit region E");
  static_assert(2 * 32 * SO * 2 <= szE, "output staging does not fit the kb buffer");
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
  static_assert(oQg % 16 == 0 && oKb % 16 == 0 && oZ % 16 == 0 && oAcm % 16 == 0 && oKt % 16 == 0 &&
                    oCst % 16 == 0 && oBt % 16 == 0 && oT % 16 == 0 && oTd % 16 == 0,
                "alignment");
};

template <int DK, int DVS, int GM>
__global__ __launch_bounds__(64 * (pipe_ncw<DVS>() + 6)) void chan_fwd_kernel(ChunkParams p) {
  constexpr int NCW = pipe_ncw<DVS>();
  constexpr int NB = DVS / (16 * NCW);
  using L = ChanLay<DK, DVS>;
  constexpr int SE = L::SE, SKT = L::SKT, SC = L::SC, SZ = L::SZ, SO = L::SO, TDS = L::TDS, TDB = L::TDB,
                SW = L::SW;
  constexpr int NKS = DK / 32;
  constexpr bool erase_ch = Gates<GM>::ERASE_CH, write_ch = Gates<GM>::WRITE_CH;

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  bf16* sEb = reinterpret_cast<bf16*>(smem + L::oEb);
  bf16* sQg = reinterpret_cast<bf16*>(smem + L::oQg);
  bf16* sKb = reinterpret_cast<bf16*>(smem + L::oKb);
  bf16* sXe = reinterpret_cast<bf16*>(smem + L::oXe);
  bf16* sXq = reinterpret_cast<bf16*>(smem + L::oXq);
  bf16* sZ = reinterpret_cast<bf16*>(smem + L::oZ);
  bf16* sAcm = reinterpret_cast<bf16*>(smem + L::oAcm);
  bf16* sAqk = reinterpret_cast<bf16*>(smem + L::oAqk);
  bf16* sKt = reinterpret_cast<bf16*>(smem + L::oKt);
  float* sCst = reinterpret_cast<float*>(smem + L::oCst);
  auto sEs = [&](int n) { return sCst + ((n & 1) ? 16 * DK : 0); };  // exp(G_sJ)
  float* sF = sCst + 4 * DK;    // exp(G_C - G_sJ)
  float* sD = sCst + 8 * DK;    // d_IJ
  float* sSc = sCst + 14 * DK;  // gamma_C, by chunk parity
  float* sBt = reinterpret_cast<float*>(smem + L::oBt);
  bf16* sT = reinterpret_cast<bf16*>(smem + L::oT);
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  int* sFlag = reinterpret_cast<int*>(sTd + 16);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  int wid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int NS = p.nslices;
  const int bh = wid / NS, slice = wid - bh * NS;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H, DV = p.DV;
  const int vbase = slice * DVS;
  const int nchunks = (T + CH - 1) / CH;
  const bool qmix = p.qmix != 0;
  const float lam = qmix ? p.lam[hh] : 0.f;
  const size_t seq0 = (size_t)bb * T * H + hh;

  // A and A_qk: blocks above the diagonal are never written and stay zero
  {
    uint4* z = reinterpret_cast<uint4*>(smem + L::oAcm);
    for (int e = tid; e < (2 * CH * SC * 2) / 16; e += 64 * (NCW + 6)) z[e] = uint4{0u, 0u, 0u, 0u};
    if (tid < 2) sFlag[tid] = 0;
  }
  __syncthreads();

  // ---- T and A_qk tiles (phase 2), shared by the producer waves ------------
  // Diagonal blocks of T go to fp32 rows for the solve, the others to bf16
  // rows; A_qk is held until phase 3.  Chunks whose block windows exceed the
  // limit take the exact tiles, staged in region E (free in phase 2).
  const bf16* qg = reinterpret_cast<const bf16*>(p.q) + seq0 * DK;
  const bf16* kg = reinterpret_cast<const bf16*>(p.k) + seq0 * DK;
  const float* g_seq = p.g + seq0 * DK;
  const float* beta_seq = p.beta ? p.beta + seq0 : nullptr;
  const float* b_seq = erase_ch ? p.b + seq0 * DK : nullptr;
  auto gram = [&](auto tiles, int n, f32x4* aqk_hold) __attribute__((always_inline)) {
    using TL = decltype(tiles);
    constexpr int NT = TL::n;
    f32x4 accT[NT], accA[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) accT[t] = accA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (sFlag[n & 1] != n + 1) {
      gram_bounded_tiles<DK, SE>(tiles, sKb, sXe, sXq, sD, accT, accA, g, l16);
    } else {
      float* st = reinterpret_cast<float*>(smem + L::oEb) + (wave - NCW) * (CH * 4 * SW);  // [t][4][SW]
      gram_exact_tiles<DK, SW, erase_ch>(tiles, st, kg, qg, g_seq, b_seq, beta_seq, qmix, lam, n, T, H, accT, accA,
                                         lane, g, l16);
    }
    gram_mask_tiles<SC, TDS, TDB>(tiles, accT, accA, aqk_hold, sT, sTd, g, l16);
  };
  auto store_aqk = [&](auto tiles, const f32x4* aqk_hold) __attribute__((always_inline)) {
    using TL = decltype(tiles);
#pragma unroll
    for (int t = 0; t < TL::n; ++t) {
      const int i = 16 * TL::I(t) + l16, j0 = 16 * TL::J(t) + 4 * g;
      *reinterpret_cast<bf16x4*>(sAqk + i * SC + j0) = cvt4(aqk_hold[t]);
    }
  };

  if (wave < NCW) {
    // =================== consumers ===========================================
    const int cw0 = 16 * NB * wave;
    f32x4 S[2 * NKS][NB];
#pragma unroll
    for (int m = 0; m < NKS; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 32 * m + 8 * g + 4 * h + r;
            const int v = vbase + cw0 + 16 * nb + l16;
            S[2 * m + h][nb][r] = p.state_in ? p.state_in[((size_t)bh * DK + c) * DV + v] : 0.f;
          }
    bf16* og = reinterpret_cast<bf16*>(p.o) + seq0 * DV + vbase;
    bf16* stage = sKb + wave * (16 * NB) * SO;  // O staging (phase 3), this wave's columns

    // the producers' prologue (block sums and constants of chunk 0) and step 0
    __syncthreads();
    __syncthreads();
    __syncthreads();
    __syncthreads();
    __syncthreads();
    for (int n = 0; n < nchunks; ++n) {
      // ---- phase 1: E_bar S and Q_gamma S ---------------------------------
      f32x4 ES[4][NB], QS[4][NB];
      {
        bf16x8 Sb[NKS][NB];
#pragma unroll
        for (int m = 0; m < NKS; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Sb[m][nb] = cat8(cvt4(S[2 * m][nb]), cvt4(S[2 * m + 1][nb]));
        bf16x8 ef[2][NKS], qf[2][NKS];
        auto load_eq = [&](int I, int slot) __attribute__((always_inline)) {
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
            ef[slot][m] = *reinterpret_cast<const bf16x8*>(sEb + (16 * I + l16) * SE + 32 * m + 8 * g);
            qf[slot][m] = *reinterpret_cast<const bf16x8*>(sQg + (16 * I + l16) * SE + 32 * m + 8 * g);
          }
        };
        load_eq(0, 0);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I < 3) load_eq(I + 1, (I + 1) & 1);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            ES[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            QS[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
              ES[I][nb] = mma32(ef[I & 1][m], Sb[m][nb], ES[I][nb]);
              QS[I][nb] = mma32(qf[I & 1][m], Sb[m][nb], QS[I][nb]);
            }
          }
        }
      }
      __syncthreads();

      // ---- phase 2: W = A (Z - E_bar S), O = Q_gamma S + A_qk W ------------
      f32x4 Wt[4][NB], Oh[4][NB];
      {
        bf16x8 Rb[2][NB];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4 R2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int I = 2 * pp + h;
              const f32x4 z = cvtf4(
                  lds_tr4(sZ + (16 * I + 4 * g + (l16 >> 2)) * SZ + cw0 + 16 * nb + 4 * (l16 & 3)));
              R2[h] = z - ES[I][nb];
            }
            Rb[pp][nb] = cat8(cvt4(R2[0]), cvt4(R2[1]));
          }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m2 = 0; m2 <= pp; ++m2) {
              const int col = 32 * pp + 8 * (l16 & 3) + 4 * h;
              const bf16x8 af = cat8(lds_tr4(sAcm + (32 * m2 + 4 * g + (l16 >> 2)) * SC + col),
                                     lds_tr4(sAcm + (32 * m2 + 16 + 4 * g + (l16 >> 2)) * SC + col));
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) acc[nb] = mma32(af, Rb[m2][nb], acc[nb]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Wt[2 * pp + h][nb] = acc[nb];
          }
        bf16x8 Wb[2][NB];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Wb[pp][nb] = cat8(cvt4(Wt[2 * pp][nb]), cvt4(Wt[2 * pp + 1][nb]));
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Oh[I][nb] = QS[I][nb];
#pragma unroll
          for (int pp = 0; pp <= I / 2; ++pp) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(sAqk + (16 * I + l16) * SC + 32 * pp + 8 * g);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Oh[I][nb] = mma32(af, Wb[pp][nb], Oh[I][nb]);
          }
        }
      }
      __syncthreads();

      // ---- phase 3: S = Diag(gamma_C) S + K_tail^T W; outputs ---------------
      {
        const float* gC = sSc + (n & 1) * DK;
        bf16x8 Wtb[2][NB];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Wtb[pp][nb] = cat8(cvt4(Wt[2 * pp][nb]), cvt4(Wt[2 * pp + 1][nb]));
        bf16x8 kt[2][2];
        auto load_kt = [&](int j, int slot) __attribute__((always_inline)) {
          const int col = 32 * (j >> 1) + 8 * (l16 & 3) + 4 * (j & 1);
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
            kt[slot][pp] = cat8(lds_tr4(sKt + (32 * pp + 8 * g + (l16 >> 2)) * SKT + col),
                                lds_tr4(sKt + (32 * pp + 8 * g + 4 + (l16 >> 2)) * SKT + col));
        };
        load_kt(0, 0);
#pragma unroll
        for (int j = 0; j < 2 * NKS; ++j) {
          if (j + 1 < 2 * NKS) load_kt(j + 1, (j + 1) & 1);
          // rows of state tile j: channels 32 (j/2) + 8 g + 4 (j%2) + r
          const f32x4 gc = *reinterpret_cast<const f32x4*>(gC + 32 * (j >> 1) + 8 * g + 4 * (j & 1));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4 acc = S[j][nb] * gc;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) acc = mma32(kt[j & 1][pp], Wtb[pp][nb], acc);
            S[j][nb] = acc;
          }
        }
        // outputs through this wave's staging: [value column][token], then
        // 8 columns of one token per lane and store
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<bf16x4*>(stage + (16 * nb + l16) * SO + 16 * I + 4 * g) = cvt4(Oh[I][nb]);
        asm volatile("" ::: "memory");  // keep the transposing reads below the stores
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
          const bf16* src = stage + (8 * k + (l16 >> 2)) * SO + 16 * g + 4 * (l16 & 3);
          const bf16x8 v = cat8(lds_tr4(src), lds_tr4(src + 4 * SO));
          const int t = n * CH + 16 * g + l16;
          if (t < T) *reinterpret_cast<bf16x8*>(og + t * H * DV + cw0 + 8 * k) = v;
        }
      }
      __syncthreads();
    }
    if (p.state_out) {
#pragma unroll
      for (int m = 0; m < NKS; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = 32 * m + 8 * g + 4 * h + r;
              const int v = vbase + cw0 + 16 * nb + l16;
              p.state_out[((size_t)bh * DK + c) * DV + v] = S[2 * m + h][nb][r];
            }
    }
  } else if (wave < NCW + 4) {
    // =================== elementwise waves ===================================
    // Wave w owns the 16-token block w of every chunk: thread = 8 key channels
    // x TT tokens, lanes along the channels (coalesced rows).
    //   phase 1  the bounded factors kb, xe, xq of its rows to LDS, K_tail
    //            in registers; K_tail of the previous chunk to LDS
    //   phase 2  prefix sums of the next chunk's log-decay inside block w; the
    //            diagonal tile (w, w) of T and A_qk
    //   phase 3  E_bar = xe Es_w, Q_gamma = xq Es_w and Z of its rows to LDS;
    //            erase vectors of the next chunk
    // Log-decays are carried in base-2 units (times log2 e), so that every
    // exponential is one exp2.
    const int w = wave - NCW, pt = tid - 64 * NCW;
    constexpr int CG = DK / 8, TG = 256 / CG, TT = CH / TG, NQ = 64 / CG;
    static_assert(TT * NQ == 16, "one 16-token block per elementwise wave");
    const int c0 = (pt % CG) * 8, tq0 = (pt / CG) * TT;  // tokens of block w
    const int qg_ = lane / CG;                            // token group inside the block
    // v layout (as the scalar-decay kernel)
    constexpr int VG = DVS / 8, VTG = 256 / VG, VPT = (CH + VTG - 1) / VTG;
    const int vv0 = (pt % VG) * 8, vtq0 = (pt / VG) * VPT;
    const bool vact = vtq0 < CH;
    constexpr float LOG2E = 1.4426950408889634f;

    const bf16* vg = reinterpret_cast<const bf16*>(p.v) + seq0 * DV + vbase;
    const float* w_seq = write_ch ? p.w + seq0 * DV + vbase : nullptr;

    // prefetched inputs of the next chunk (v and the write gate: of the
    // current one), at token indices clamped to T - 1
    bf16x8 rk[TT], rq[TT];
    f32x4 rg[TT][2], rb[erase_ch ? TT : 1][2];
    float rbeta[erase_ch ? 1 : TT];
    bf16x8 rv[VPT];
    f32x4 rw[write_ch ? VPT : 1][2];
    float rvb[write_ch ? 1 : VPT];
    bf16x8 re[TT];          // erase vectors e of the next chunk (bf16)
    bf16x8 ktail[TT];       // K_tail rows of the current chunk, stored one step later
    // Loads address the chunk from a uniform base with 32-bit per-lane byte
    // offsets (row of the token within the chunk), so that they take the
    // scalar-base form and keep no 64-bit addresses in vector registers.
    auto ldg = [&](auto vt, const void* base, unsigned byteoff) __attribute__((always_inline)) {
      using V = decltype(vt);
      return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byteoff);
    };
    // token rows (t * H) of my tokens relative to the chunk start
    auto row = [&](int n, int t) __attribute__((always_inline)) -> unsigned {
      return (unsigned)(min(n * CH + t, T - 1) - n * CH) * H;
    };
    auto load_g = [&](int n) __attribute__((always_inline)) {
      const size_t cb = (size_t)n * CH * H * DK;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const unsigned o = row(n, tq0 + u) * DK + c0;
        rg[u][0] = ldg(f32x4{}, g_seq + cb, 4 * o);
        rg[u][1] = ldg(f32x4{}, g_seq + cb, 4 * o + 16);
      }
    };
    auto load_kqb = [&](int n) __attribute__((always_inline)) {
      const size_t cb = (size_t)n * CH * H * DK;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const unsigned r = row(n, tq0 + u), o = r * DK + c0;
        rk[u] = ldg(bf16x8{}, kg + cb, 2 * o);
        rq[u] = ldg(bf16x8{}, qg + cb, 2 * o);
        if constexpr (erase_ch) {
          rb[u][0] = ldg(f32x4{}, b_seq + cb, 4 * o);
          rb[u][1] = ldg(f32x4{}, b_seq + cb, 4 * o + 16);
        } else {
          rbeta[u] = ldg(float{}, beta_seq + (size_t)n * CH * H, 4 * r);
        }
      }
    };
    auto load_v = [&](int n) __attribute__((always_inline)) {
      if (!vact) return;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const unsigned r = row(n, vtq0 + u);
        const unsigned o = r * DV + vv0;
        rv[u] = ldg(bf16x8{}, vg + (size_t)n * CH * H * DV, 2 * o);
        if constexpr (write_ch) {
          const float* wc = w_seq + (size_t)n * CH * H * DV;
          rw[u][0] = ldg(f32x4{}, wc, 4 * o);
          rw[u][1] = ldg(f32x4{}, wc, 4 * o + 16);
        } else {
          rvb[u] = ldg(float{}, beta_seq + (size_t)n * CH * H, 4 * r);
        }
      }
    };

    // ---- phase 2 of the previous step: in-block prefix sums ------------------
    // Hl = prefix sums over my TT tokens; Hsx = (sum at the block's first
    // token) - (sum over the token groups before mine), so that the decay of
    // token u relative to the block start is dl = Hsx - Hl[u] >= 0.
    float Hl[TT][8], Hsx[8];
    auto scan = [&](int n) __attribute__((always_inline)) {
      if (n * CH + CH > T) {
        // last chunk: g = 0 past the end
#pragma unroll
        for (int u = 0; u < TT; ++u)
          if (n * CH + tq0 + u >= T) rg[u][0] = rg[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float excl[8], tot[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < TT; ++u) {
          sum += (i < 4 ? rg[u][0][i] : rg[u][1][i - 4]) * LOG2E;
          Hl[u][i] = sum;
        }
        tot[i] = sum;
        // exclusive prefix over the token groups (lanes CG apart)
        float x = sum;
#pragma unroll
        for (int d = CG; d < 64; d *= 2) {
          const float y = __shfl_up(x, d);
          x += lane >= d ? y : 0.f;
        }
        excl[i] = x - sum;
      }
      if (qg_ == 0) st8(sBt + w * DK + c0, Hl[0]);
      if (qg_ == NQ - 1) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = excl[i] + tot[i];
        st8(sBt + (4 + w) * DK + c0, e);
      }
      // (one wave: its row is complete before this read)
      const V8<float> hs = ld8(sBt + w * DK + c0);
      bool bad = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Hsx[i] = hs[i] - excl[i];
        bad |= !(Hsx[i] - Hl[TT - 1][i] <= WINDOW_LIMIT * LOG2E);
      }
      // a block window above the limit switches the chunk to the exact Gram
      if (bad) sFlag[n & 1] = n + 1;
    };

    // erase vectors of the next chunk once its loads have landed: e = b k or
    // beta (k + lam q) (lam = 0 without the Q-Delta mix); k = q = 0 past the
    // end
    auto erase_rows = [&](int n) __attribute__((always_inline)) {
      if (n * CH + CH > T) {
#pragma unroll
        for (int u = 0; u < TT; ++u)
          if (n * CH + tq0 + u >= T) rk[u] = rq[u] = bf16x8{};
      }
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        f32x4 lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (erase_ch) {
            lo[i] = rb[u][0][i] * (float)rk[u][i];
            hi[i] = rb[u][1][i] * (float)rk[u][i + 4];
          } else {
            lo[i] = rbeta[u] * __builtin_fmaf(lam, (float)rq[u][i], (float)rk[u][i]);
            hi[i] = rbeta[u] * __builtin_fmaf(lam, (float)rq[u][i + 4], (float)rk[u][i + 4]);
          }
        }
        re[u] = cat8(cvt4(lo), cvt4(hi));
      }
    };

    // ---- phase 1 ---------------------------------------------------------------
    // gamma_C = 2^G_C (wave 0; G_C = sum of the block totals), then the
    // bounded factors of my rows and K_tail = kb f_w (f_w from the Gram wave
    // 1, one phase earlier).
    constexpr int CPL = DK / 64;
    auto prep = [&](auto wc, int n) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      if constexpr (W == 0) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          const int c = CPL * lane + e;
          float gc = 0.f;
#pragma unroll
          for (int J = 0; J < 4; ++J) gc += sBt[(4 + J) * DK + c];
          sSc[(n & 1) * DK + c] = __builtin_amdgcn_exp2f(gc);
        }
      }
      const V8<float> fk = ld8(sF + W * DK + c0);
      const bool bad = sFlag[n & 1] == n + 1;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int t = tq0 + u;
        float kb[8], xe[8], xq[8], kt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float kv = (float)rk[u][i];
          const float qv = (float)rq[u][i];
          const float ev = (float)re[u][i];
          const float dl = Hsx[i] - Hl[u][i];  // >= 0
          const float ir = __builtin_amdgcn_exp2f(-dl);
          kb[i] = kv * __builtin_amdgcn_exp2f(dl);
          xe[i] = ev * ir;
          xq[i] = qv * ir;
          kt[i] = kb[i] * fk[i];  // k exp(G_C - G) <= |k|
        }
        if (bad) {
          // kb may have overflowed (the chunk takes the exact Gram): K_tail
          // from its own exponent, G_C - G = (G_C - G_sw) + dl
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float lf = -sBt[W * DK + c0 + i];
#pragma unroll
            for (int J = W; J < 4; ++J) lf += sBt[(4 + J) * DK + c0 + i];
            kt[i] = (float)rk[u][i] * __builtin_amdgcn_exp2f(lf + Hsx[i] - Hl[u][i]);
          }
        }
        st8(sKb + t * SE + c0, kb);
        st8(sXe + t * SE + c0, xe);
        st8(sXq + t * SE + c0, xq);
        ktail[u] = cat8(cvt4(f32x4{kt[0], kt[1], kt[2], kt[3]}), cvt4(f32x4{kt[4], kt[5], kt[6], kt[7]}));
        // (one token at a time: no scheduling barrier needed here)
      }
    };

    auto store_ktail = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < TT; ++u) *reinterpret_cast<bf16x8*>(sKt + (tq0 + u) * SKT + c0) = ktail[u];
    };

    // ---- phase 3: E_bar = xe Es_w, Q_gamma = xq Es_w of my rows; Z = gate * v --
    auto finish = [&](int n) __attribute__((always_inline)) {
      const int t0 = n * CH;
      const V8<float> es = ld8(sEs(n) + w * DK + c0);
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int t = tq0 + u;
        const bf16x8 xe = *reinterpret_cast<const bf16x8*>(sXe + t * SE + c0);
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(sXq + t * SE + c0);
        f32x4 a0, a1, b0, b1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[i] = (float)xe[i] * es[i];
          a1[i] = (float)xe[i + 4] * es[i + 4];
          b0[i] = (float)xq[i] * es[i];
          b1[i] = (float)xq[i + 4] * es[i + 4];
        }
        *reinterpret_cast<bf16x8*>(sEb + t * SE + c0) = cat8(cvt4(a0), cvt4(a1));
        *reinterpret_cast<bf16x8*>(sQg + t * SE + c0) = cat8(cvt4(b0), cvt4(b1));
      }
      if (vact) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int t = vtq0 + u;
          const bool ok = t0 + t < T;
          float z[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float gate;
            if constexpr (write_ch) gate = e < 4 ? rw[u][0][e] : rw[u][1][e - 4];
            else gate = rvb[u];
            z[e] = ok ? gate * (float)rv[u][e] : 0.f;
          }
          st8(sZ + t * SZ + vv0, z);
        }
      }
    };

    auto elementwise_loop = [&](auto wc) __attribute__((always_inline)) {
      if (nchunks > 0) {
        load_g(0);
        load_kqb(0);
        scan(0);
        erase_rows(0);
        load_g(min(1, nchunks - 1));
      }
      __syncthreads();  // block sums of chunk 0 to the Gram wave 1
      __syncthreads();  // its constants of chunk 0 to every wave
      // Every step runs the same code: the next chunk's index is clamped, so
      // the last step repeats harmless work on the last chunk, and every
      // prefetched register is written in the step that reads it (with
      // conditional loads the compiler keeps them all live across steps).
      // Loads are spread over the phases (v in phase 1, k, q and the erase
      // gate in phase 2, the log-decay in phase 3), so that a step's requests
      // do not leave in one burst that stalls the issuing waves.
      constexpr int W = decltype(wc)::value;
      f32x4 aqk_hold[1];
      for (int n = 0; n < nchunks; ++n) {
        const int nn = min(n + 1, nchunks - 1), nn2 = min(n + 2, nchunks - 1);
        // phase 1
        if (n > 0) store_ktail();
        prep(wc, n);
        // the loads stay behind the factors: hoisted into them they would
        // add to the registers held
        __builtin_amdgcn_sched_barrier(0);
        load_v(n);
        __syncthreads();
        // phase 2
        load_kqb(nn);
        scan(nn);
        gram(TileList<W, W>{}, n, aqk_hold);
        __syncthreads();
        // phase 3
        store_aqk(TileList<W, W>{}, aqk_hold);
        finish(n);
        load_g(nn2);
        erase_rows(nn);
        __syncthreads();
      }
      // last step: the consumers apply the last chunk
      if (nchunks > 0) store_ktail();
      __syncthreads();
      __syncthreads();
      __syncthreads();
    };
    switch (w) {
      case 0: elementwise_loop(IC<0>{}); break;
      case 1: elementwise_loop(IC<1>{}); break;
      case 2: elementwise_loop(IC<2>{}); break;
      default: elementwise_loop(IC<3>{}); break;
    }
  } else {
    // =================== Gram waves ==========================================
    // phase 2: the T and A_qk tiles below the diagonal blocks; phase 3: wave
    // 0 inverts I + T, wave 1 forms the per-(block, channel) constants of the
    // next chunk, both store A_qk.
    const int gw = wave - NCW - 4;

    // Constants of chunk n from its block sums, for the DK / 64 channels of
    // each lane (base 2): P_J = G before block J, G_sJ = P_J + Bt[J],
    // G_C = P_4; Es_J = 2^G_sJ, f_J = 2^(G_C - G_sJ), d_IJ = 2^(G_sI - G_sJ).
    constexpr int CPL = DK / 64;
    auto table = [&](int n) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const int c = CPL * lane + e;
        float P[5], gs[4];
        P[0] = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          gs[J] = P[J] + sBt[J * DK + c];
          P[J + 1] = P[J] + sBt[(4 + J) * DK + c];
        }
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          sEs(n)[J * DK + c] = __builtin_amdgcn_exp2f(gs[J]);
          sF[J * DK + c] = __builtin_amdgcn_exp2f(P[4] - gs[J]);
        }
#pragma unroll
        for (int I = 1; I < 4; ++I)
#pragma unroll
          for (int J = 0; J < I; ++J) sD[(I * (I - 1) / 2 + J) * DK + c] = __builtin_amdgcn_exp2f(gs[I] - gs[J]);
      }
    };

    f32x4 aqk_hold[3];
    auto gram_loop = [&](auto gc, auto tiles) __attribute__((always_inline)) {
      constexpr int G = decltype(gc)::value;
      __syncthreads();  // (the elementwise waves' block sums of chunk 0)
      if constexpr (G == 1) {
        if (nchunks > 0) table(0);
      }
      __syncthreads();
      for (int n = 0; n < nchunks; ++n) {
        __syncthreads();
        gram(tiles, n, aqk_hold);
        __syncthreads();
        if constexpr (G == 0) solve_inverse<SC, TDS, TDB>(sTd, sT, sAcm, g, l16);
        store_aqk(tiles, aqk_hold);
        // constants of the next chunk (its block sums came in phase 2)
        if constexpr (G == 1) {
          if (n + 1 < nchunks) table(n + 1);
        }
        __syncthreads();
      }
      __syncthreads();
      __syncthreads();
      __syncthreads();
    };
    // the six tiles below the diagonal (the decay-scaled ones), three each;
    // tiles sharing a row block I share its xe and xq fragments
    if (gw == 0) gram_loop(IC<0>{}, TileList<1, 0, 3, 0, 3, 1>{});
    else gram_loop(IC<1>{}, TileList<2, 0, 2, 1, 3, 2>{});
  }
}

template <int DK, int DVS>
constexpr int chan_lds_bytes() {
  return ChanLay<DK, DVS>::TOTAL;
}

}  // namespace gdr
