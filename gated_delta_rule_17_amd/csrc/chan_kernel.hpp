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
// Workgroup: consumer waves as in pipe_kernel.hpp plus 4 producer waves, one
// chunk step = three barriers.  The per-chunk operands do not fit twice in
// LDS, so each has one buffer, written in the phase after its last reader:
//   region   written by producers      read by consumers
//   E        phase 3 (E_bar, Q_gamma)  phase 1 (K S, Q S)
//   P        phase 1 (kb, xe, xq)      -           (producer Gram, phase 2;
//                                                   consumer O staging, phase 3)
//   C        phase 3 (Z, A, A_qk)      phase 2 (W, O)
//   K        phase 1 of the next step  phase 3 (state update)
//            (K_tail)
// Region E is free in phase 2 and holds the exact-Gram staging when needed.
#pragma once

#include "chunk_kernel.hpp"
#include "pipe_kernel.hpp"

namespace gdr {

template <int DK, int DVS>
struct ChanLay {
  static constexpr int SE = DK + 8;                       // rows of E_bar, Q_gamma, kb, xe, xq
  static constexpr int SKT = DK + (DK == 128 ? 32 : 24);  // K_tail rows (transposing reads)
  static constexpr int SC = CH + 8, SZ = DVS + 8, SO = CH + 8;
  static constexpr int TDS = 20, TDB = 16 * TDS;
  static constexpr int SW = DK / 16;  // channels per slab of the exact Gram
  static constexpr int szE = CH * SE * 2;
  static constexpr int oEb = 0, oQg = oEb + szE;                            // region E
  static constexpr int oKb = oQg + szE, oXe = oKb + szE, oXq = oXe + szE;  // region P
  static constexpr int oZ = oXq + szE;                                     // region C
  static constexpr int oAcm = oZ + CH * SZ * 2;
  static constexpr int oAqk = oAcm + CH * SC * 2;
  static constexpr int oKt = oAqk + CH * SC * 2;  // region K
  static constexpr int oSc = oKt + CH * SKT * 2;  // 2 x gamma_C [DK] fp32 (chunk parity)
  static constexpr int oD = oSc + 2 * DK * 4;     // d_IJ [6][DK] fp32
  static constexpr int oEs = oD + 6 * DK * 4;     // exp(G at block starts) [4][DK] fp32
  static constexpr int oT = oEs + 4 * DK * 4;     // T below the diagonal, bf16 rows
  static constexpr int oTd = oT + CH * SC * 2;    // diagonal blocks of T, fp32 rows
  static constexpr int oFlag = oTd + 4 * TDB * 4;
  static constexpr int TOTAL = oFlag + 16;
  static_assert(4 * CH * 4 * SW * 4 <= 2 * szE, "exact-Gram staging does not fit region E");
  static_assert(2 * 32 * SO * 2 <= szE, "output staging does not fit the kb buffer");
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
  static_assert(oQg % 16 == 0 && oKb % 16 == 0 && oZ % 16 == 0 && oAcm % 16 == 0 && oKt % 16 == 0 &&
                    oSc % 16 == 0 && oD % 16 == 0 && oT % 16 == 0 && oTd % 16 == 0,
                "alignment");
};

template <int DK, int DVS, int GM>
__global__ __launch_bounds__(64 * (pipe_ncw<DVS>() + 4)) void chan_fwd_kernel(ChunkParams p) {
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
  float* sSc = reinterpret_cast<float*>(smem + L::oSc);
  float* sD = reinterpret_cast<float*>(smem + L::oD);
  float* sEs = reinterpret_cast<float*>(smem + L::oEs);
  bf16* sT = reinterpret_cast<bf16*>(smem + L::oT);
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  int* sFlag = reinterpret_cast<int*>(smem + L::oFlag);

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
    for (int e = tid; e < (2 * CH * SC * 2) / 16; e += 64 * (NCW + 4)) z[e] = uint4{0u, 0u, 0u, 0u};
    if (tid == 0) *sFlag = 0;
  }
  __syncthreads();

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
  } else {
    // =================== producers ===========================================
    // Phase 1: cumulative log-decay per key channel and the bounded factors
    // kb, xe, xq (rows to LDS), d_IJ and exp(G) at the block starts, gamma_C;
    // K_tail of the previous chunk to LDS.  Phase 2: T and A_qk tiles.
    // Phase 3: wave 0 inverts I + T; every wave stores its A_qk tiles and its
    // rows of E_bar, Q_gamma and Z.
    const int pw = wave - NCW, pt = tid - 64 * NCW;
    // factor layout: thread = 8 key channels x TT tokens; the SEG token groups
    // of a channel group are consecutive lanes of one wave, so the per-channel
    // prefix sum runs across lanes without a barrier
    constexpr int CGN = DK / 8, SEG = 256 / CGN, TT = CH / SEG;
    static_assert(SEG == 16 || SEG == 32, "prefix-sum segment");
    const int tg = lane % SEG, cg = pw * (64 / SEG) + lane / SEG;
    const int c0 = 8 * cg, tq0 = TT * tg;
    const int segbase = lane - tg;
    // x at lane SRC of this lane's segment: a DPP row broadcast when the
    // segment is one 16-lane row, else a lane permute
    auto seg_lane = [&](auto src, float x) __attribute__((always_inline)) -> float {
      constexpr int SRC = decltype(src)::value;
      if constexpr (SEG == 16)
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + SRC,
                                                                      0xf, 0xf, false));
      else
        return __shfl(x, segbase + SRC);
    };
    const int myJ = tq0 / 16;  // 16-token block of my tokens
    // v layout (as the scalar-decay kernel)
    constexpr int VG = DVS / 8, VTG = 256 / VG, VPT = (CH + VTG - 1) / VTG;
    const int vv0 = (pt % VG) * 8, vtq0 = (pt / VG) * VPT;
    const bool vact = vtq0 < CH;

    const bf16* qg = reinterpret_cast<const bf16*>(p.q) + seq0 * DK;
    const bf16* kg = reinterpret_cast<const bf16*>(p.k) + seq0 * DK;
    const bf16* vg = reinterpret_cast<const bf16*>(p.v) + seq0 * DV + vbase;
    const float* g_seq = p.g + seq0 * DK;
    const float* beta_seq = p.beta ? p.beta + seq0 : nullptr;
    const float* b_seq = erase_ch ? p.b + seq0 * DK : nullptr;
    const float* w_seq = write_ch ? p.w + seq0 * DV + vbase : nullptr;

    // prefetched inputs of the next chunk (k, q, g: phase 1; b or beta:
    // phase 2; v and w or beta: phase 3), at token indices clamped to T - 1
    bf16x8 rk[TT], rq[TT];
    f32x4 rg[TT][2], rb[erase_ch ? TT : 1][2];
    float rbeta[erase_ch ? 1 : TT];
    bf16x8 rv[VPT];
    f32x4 rw[write_ch ? VPT : 1][2];
    float rvb[write_ch ? 1 : VPT];
    bf16x8 ktail[TT];  // K_tail rows of the current chunk, stored one step later
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
    auto load_kqg = [&](int n) __attribute__((always_inline)) {
      const size_t cb = (size_t)n * CH * H * DK;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const unsigned o = row(n, tq0 + u) * DK + c0;
        rk[u] = ldg(bf16x8{}, kg + cb, 2 * o);
        rq[u] = ldg(bf16x8{}, qg + cb, 2 * o);
        rg[u][0] = ldg(f32x4{}, g_seq + cb, 4 * o);
        rg[u][1] = ldg(f32x4{}, g_seq + cb, 4 * o + 16);
      }
    };
    auto load_b = [&](int n) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const unsigned r = row(n, tq0 + u);
        if constexpr (erase_ch) {
          const unsigned o = r * DK + c0;
          const float* bc = b_seq + (size_t)n * CH * H * DK;
          rb[u][0] = ldg(f32x4{}, bc, 4 * o);
          rb[u][1] = ldg(f32x4{}, bc, 4 * o + 16);
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

    // erase vector of my token u, channel i (fp32)
    auto erase_of = [&](int u, int i, float kv, float qv) -> float __attribute__((always_inline)) {
      if constexpr (erase_ch) return (i < 4 ? rb[u][0][i] : rb[u][1][i - 4]) * kv;
      else return rbeta[u] * (qmix ? kv + lam * qv : kv);
    };

    // ---- phase 1 ---------------------------------------------------------------
    auto prep = [&](int n) __attribute__((always_inline)) {
      const int t0 = n * CH;
      float G[TT][8];
      float tot[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < TT; ++u) {
          const float gv = (t0 + tq0 + u < T) ? (i < 4 ? rg[u][0][i] : rg[u][1][i - 4]) : 0.f;
          s += gv;
          G[u][i] = s;
        }
        tot[i] = s;
      }
      // exclusive prefix of the per-thread totals over the segment
      float GC[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = tot[i];
#define GDR_SEG_ADD(ctrl, rmask)                                                                    \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rmask, \
                                                              0xf, false))
        GDR_SEG_ADD(0x111, 0xf);  // row_shr:1
        GDR_SEG_ADD(0x112, 0xf);  // row_shr:2
        GDR_SEG_ADD(0x114, 0xf);  // row_shr:4
        GDR_SEG_ADD(0x118, 0xf);  // row_shr:8
        if constexpr (SEG == 32) GDR_SEG_ADD(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
#undef GDR_SEG_ADD
        const float excl = x - tot[i];
#pragma unroll
        for (int u = 0; u < TT; ++u) G[u][i] += excl;
        GC[i] = seg_lane(IC<SEG - 1>{}, x);
      }
      // G at the start of my block; d_IJ = exp(G_{s_I} - G_{s_J}) for the
      // blocks J before mine (stored by the lanes that hold a block start)
      const bool bstart = tq0 % 16 == 0;
      float Gm[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float g0 = seg_lane(IC<0>{}, G[0][i]), g1 = seg_lane(IC<16 / TT>{}, G[0][i]),
                    g2 = seg_lane(IC<32 / TT>{}, G[0][i]), g3 = seg_lane(IC<48 / TT>{}, G[0][i]);
        Gm[i] = myJ == 0 ? g0 : (myJ == 1 ? g1 : (myJ == 2 ? g2 : g3));
      }
      auto dblock = [&](auto Jc) __attribute__((always_inline)) {
        constexpr int J = decltype(Jc)::value;
        float d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = fexp(Gm[i] - seg_lane(IC<16 * J / TT>{}, G[0][i]));
        if (bstart && J < myJ) st8(sD + (myJ * (myJ - 1) / 2 + J) * DK + c0, d);
      };
      dblock(IC<0>{});
      dblock(IC<1>{});
      dblock(IC<2>{});
      // block windows above the limit switch this chunk to the exact Gram
      bool bad = false;
#pragma unroll
      for (int u = 0; u < TT; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) bad |= !(Gm[i] - G[u][i] <= WINDOW_LIMIT);
      if (bad) *sFlag = n + 1;
      if (bstart) {
        float es[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) es[i] = fexp(Gm[i]);
        st8(sEs + myJ * DK + c0, es);
      }
      if (tg == 0) {
        float gc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gc[i] = fexp(GC[i]);
        st8(sSc + (n & 1) * DK + c0, gc);
      }
      // bounded factors, and K_tail (kept in registers for one step)
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int t = tq0 + u;
        const bool ok = t0 + t < T;
        float kb[8], xe[8], xq[8], kt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float kv = ok ? (float)rk[u][i] : 0.f;
          const float qv = ok ? (float)rq[u][i] : 0.f;
          const float ev = erase_of(u, i, kv, qv);
          const float dl = Gm[i] - G[u][i];  // >= 0
          const float ir = fexp(-dl);
          kb[i] = kv * fexp(dl);
          xe[i] = ev * ir;
          xq[i] = qv * ir;
          kt[i] = kv * fexp(GC[i] - G[u][i]);  // <= |k|
        }
        st8(sKb + t * SE + c0, kb);
        st8(sXe + t * SE + c0, xe);
        st8(sXq + t * SE + c0, xq);
        f32x4 lo = {kt[0], kt[1], kt[2], kt[3]}, hi = {kt[4], kt[5], kt[6], kt[7]};
        ktail[u] = cat8(cvt4(lo), cvt4(hi));
        __builtin_amdgcn_sched_barrier(0);  // one token's temporaries at a time
      }
    };

    auto store_ktail = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < TT; ++u) *reinterpret_cast<bf16x8*>(sKt + (tq0 + u) * SKT + c0) = ktail[u];
    };

    // Exact T and A_qk entries for chunks whose block windows exceed the
    // limit: every lane accumulates its four entries (i, j) of each tile as
    // sum_c x_i[c] k_j[c] exp(G_i[c] - G_j[c]) in fp32, over slabs of SW
    // channels staged by this wave alone (region E, free in phase 2).
    auto gram_exact = [&](auto tl, int n, f32x4* accT, f32x4* accA) __attribute__((always_inline)) {
      using TL = decltype(tl);
      float* st = reinterpret_cast<float*>(smem + L::oEb) + pw * (CH * 4 * SW);  // [t][4][SW]
      const int t0 = n * CH;
      const int t = lane;  // staging: one token per lane
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
          if constexpr (erase_ch) ev = (ok ? b_seq[a] : 0.f) * kv;
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
    };

    // ---- phase 2: T and A_qk tiles --------------------------------------------
    // Tiles as in the scalar-decay kernel: wave 0: (3,0) (3,1) (0,0); wave 1:
    // (2,0) (2,1) (2,2); wave 2: (1,0) (1,1); wave 3: (3,2) (3,3), both
    // kinds, computed transposed (D^T = kb_J X_I^T).
    f32x4 aqk_hold[3];
    auto gram = [&](auto tiles, int n) __attribute__((always_inline)) {
      using TL = decltype(tiles);
      constexpr int NT = TL::n;
      f32x4 accT[NT], accA[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) accT[t] = accA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (*sFlag != n + 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
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
          // one tile's fragments in flight at a time (register budget)
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        gram_exact(tiles, n, accT, accA);
      }
      // masks; i = row (lane), j = 4 columns
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int I = TL::I(t), J = TL::J(t);
        const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
        f32x4 xT, xA;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xT[r] = (j0 + r < i) ? accT[t][r] : 0.f;   // T: j < i
          xA[r] = (j0 + r <= i) ? accA[t][r] : 0.f;  // A_qk: j <= i
        }
        aqk_hold[t] = xA;
        if (J < I) *reinterpret_cast<bf16x4*>(sT + i * SC + j0) = cvt4(xT);
        else *reinterpret_cast<f32x4*>(sTd + I * TDB + l16 * TDS + 4 * g) = xT;
      }
    };

    // ---- phase 3 ---------------------------------------------------------------
    auto store_aqk = [&](auto tiles) __attribute__((always_inline)) {
      using TL = decltype(tiles);
#pragma unroll
      for (int t = 0; t < TL::n; ++t) {
        const int i = 16 * TL::I(t) + l16, j0 = 16 * TL::J(t) + 4 * g;
        *reinterpret_cast<bf16x4*>(sAqk + i * SC + j0) = cvt4(aqk_hold[t]);
      }
    };
    // E_bar = xe exp(G_s), Q_gamma = xq exp(G_s) for my rows; Z = gate * v
    auto finish = [&](int n) __attribute__((always_inline)) {
      const int t0 = n * CH;
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(sEs + myJ * DK + c0);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(sEs + myJ * DK + c0 + 4);
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        const int t = tq0 + u;
        const bf16x8 xe = *reinterpret_cast<const bf16x8*>(sXe + t * SE + c0);
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(sXq + t * SE + c0);
        f32x4 a0 = {(float)xe[0], (float)xe[1], (float)xe[2], (float)xe[3]};
        f32x4 a1 = {(float)xe[4], (float)xe[5], (float)xe[6], (float)xe[7]};
        f32x4 b0 = {(float)xq[0], (float)xq[1], (float)xq[2], (float)xq[3]};
        f32x4 b1 = {(float)xq[4], (float)xq[5], (float)xq[6], (float)xq[7]};
        *reinterpret_cast<bf16x8*>(sEb + t * SE + c0) = cat8(cvt4(a0 * e0), cvt4(a1 * e1));
        *reinterpret_cast<bf16x8*>(sQg + t * SE + c0) = cat8(cvt4(b0 * e0), cvt4(b1 * e1));
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


    auto producer_loop = [&](auto tiles) __attribute__((always_inline)) {
      // inputs of chunk n + 1 are requested a step ahead (k, q, g in phase 1,
      // the erase gate in phase 2); v and the write gate of chunk n, which
      // are used in phase 3, only after the prefix sum of chunk n, to keep
      // them out of its registers
      if (nchunks > 0) {
        load_kqg(0);
        load_b(0);
      }
      for (int n = 0; n <= nchunks; ++n) {
        const bool cur = n < nchunks, more = n + 1 < nchunks;
        // phase 1
        if (n > 0) store_ktail();
        if (cur) prep(n);
        // the next chunk's loads stay behind the prefix sum: hoisted into
        // it they would double the registers it holds
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_kqg(n + 1);
        if (cur) load_v(n);
        __syncthreads();
        // phase 2
        if (more) load_b(n + 1);
        if (cur) gram(tiles, n);
        __syncthreads();
        // phase 3
        if (cur) {
          if (pw == 0) solve_inverse<SC, TDS, TDB>(sTd, sT, sAcm, g, l16);
          store_aqk(tiles);
          finish(n);
        }
        __syncthreads();
      }
    };
    switch (pw) {
      case 0: producer_loop(Tiles<3, 3, 0, 3, 1, 0, 0>{}); break;
      case 1: producer_loop(Tiles<3, 2, 0, 2, 1, 2, 2>{}); break;
      case 2: producer_loop(Tiles<2, 1, 0, 1, 1>{}); break;
      default: producer_loop(Tiles<2, 3, 2, 3, 3>{}); break;
    }
  }
}

template <int DK, int DVS>
constexpr int chan_lds_bytes() {
  return ChanLay<DK, DVS>::TOTAL;
}

}  // namespace gdr
