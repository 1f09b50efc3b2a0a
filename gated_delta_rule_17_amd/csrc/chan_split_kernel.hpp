// Two-pass chunkwise forward for a per-key-channel decay (bf16 I/O, dk 128),
// for workloads with few heads: there the single-pass kernel of
// chan_kernel.hpp splits each head into many value slices, and every slice
// repeats the chunk's elementwise, Gram and solve work on its own critical
// path.  Here that work runs once per (batch, head, chunk), in parallel over
// chunks, and the per-slice recurrence only applies it.
//
// Same chunk form as chan_kernel.hpp ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", key design 2, with W = A (Z - E_bar S)):
//   pass 1 (chan_prep_kernel, one workgroup per chunk): the bounded factors
//     and block constants of the chunk, E_bar = gamma e, Q_gamma = gamma q,
//     K_tail = (gamma_C / gamma) k, the T and A_qk tiles (bounded factors, or
//     exact fp32 tiles past the window limit), A = (I + T)^{-1}, gamma_C;
//     written to one record per chunk in a caller-provided workspace
//   pass 2 (chan_rec_kernel, one workgroup per (head, value slice)): the
//     state recurrence, with loader waves copying record n + 1 into LDS
//     while the consumer waves apply record n; one barrier per chunk.
// Workspace record of a chunk (bytes; n = chunk within its sequence; records
// ordered by (batch, head, chunk)):
//   E_bar [64][dk] bf16 | Q_gamma [64][dk] bf16 | K_tail [64][dk] bf16 |
//   A column-major (Acm[j][i] = A[i][j]), its ten non-zero 16 x 16 blocks |
//   A_qk row-major, its ten non-zero blocks | gamma_C [dk] fp32
// The six blocks above the diagonal of A and A_qk are zero and not stored:
// A_qk keeps, for row block I, the blocks J <= I of its 16 rows (rows of
// 32 (I + 1) bytes, row blocks in order); Acm keeps, for row block J, the
// blocks I >= J (rows of 32 (4 - J) bytes).  Each takes 320 pieces of 16 bytes.
#pragma once

#include "chan_kernel.hpp"

namespace gdr {

template <int DK>
struct SplitRec {
  static constexpr int PIECES_A = 320;  // 16-byte pieces of the ten stored blocks
  static constexpr int oEb = 0, oQg = CH * DK * 2, oKt = 2 * CH * DK * 2;
  static constexpr int oAcm = 3 * CH * DK * 2, oAqk = oAcm + PIECES_A * 16, oGc = oAqk + PIECES_A * 16;
  static constexpr int BYTES = (oGc + DK * 4 + 255) / 256 * 256;
};

// ---- pass 1 ------------------------------------------------------------------
template <int DK>
struct PrepLay {
  static constexpr int SE = DK + 8, SC = CH + 8, TDS = 20, TDB = 16 * TDS, SW = DK / 32;
  static constexpr int szE = CH * SE * 2;
  static constexpr int oKb = 0, oXe = szE, oXq = 2 * szE;  // bounded factors; A reuses xq after the Gram
  static constexpr int oT = 3 * szE;                       // T below the diagonal blocks, bf16 rows
  static constexpr int oTd = oT + CH * SC * 2;             // diagonal blocks of T, fp32
  static constexpr int oBt = oTd + 4 * TDB * 4;            // block sums of the log-decay, 8 rows of DK
  static constexpr int oCst = oBt + 8 * DK * 4;            // exp(G_sJ) 4 rows, exp(G_C - G_sJ) 4, d_IJ 6
  static constexpr int oFlag = oCst + 14 * DK * 4;
  static constexpr int TOTAL = oFlag + 16;
  static_assert(CH * SC * 2 <= szE, "A does not fit the xq rows");
  static_assert(4 * CH * 4 * SW * 4 <= 2 * szE, "exact-Gram staging does not fit the kb and xe rows");
  static_assert(TOTAL <= 80 * 1024, "two workgroups per CU");
};

template <int DK, int GM>
__global__ __launch_bounds__(256) void chan_prep_kernel(ChunkParams p, char* __restrict__ ws) {
  using L = PrepLay<DK>;
  using R = SplitRec<DK>;
  constexpr int SE = L::SE, SC = L::SC, TDS = L::TDS, TDB = L::TDB, SW = L::SW;
  constexpr bool erase_ch = Gates<GM>::ERASE_CH;
  constexpr int CG = DK / 8, TT = CH * CG / 256;  // lane: 8 key channels x TT tokens
  static_assert(TT * (64 / CG) == 16, "one 16-token block per wave");
  constexpr float LOG2E = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  bf16* sKb = reinterpret_cast<bf16*>(smem + L::oKb);
  bf16* sXe = reinterpret_cast<bf16*>(smem + L::oXe);
  bf16* sXq = reinterpret_cast<bf16*>(smem + L::oXq);
  bf16* sA = sXq;
  bf16* sT = reinterpret_cast<bf16*>(smem + L::oT);
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  float* sBt = reinterpret_cast<float*>(smem + L::oBt);
  float* sEs = reinterpret_cast<float*>(smem + L::oCst);
  float* sF = sEs + 4 * DK;
  float* sD = sEs + 8 * DK;
  int* sFlag = reinterpret_cast<int*>(smem + L::oFlag);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 16-token block of this wave
  const int g = lane >> 4, l16 = lane & 15;
  const int T = p.T, H = p.H;
  const int nchunks = (T + CH - 1) / CH;
  const int job = blockIdx.x;  // (batch, head) major, chunk minor
  const int bh = job / nchunks, n = job - bh * nchunks;
  const int bb = bh / H, hh = bh - bb * H;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const bool qmix = p.qmix != 0;
  const float lam = qmix ? p.lam[hh] : 0.f;
  char* rec = ws + (size_t)job * R::BYTES;

  const bf16* kg = reinterpret_cast<const bf16*>(p.k) + seq0 * DK;
  const bf16* qg = reinterpret_cast<const bf16*>(p.q) + seq0 * DK;
  const float* g_seq = p.g + seq0 * DK;
  const float* beta_seq = p.beta ? p.beta + seq0 : nullptr;
  const float* b_seq = erase_ch ? p.b + seq0 * DK : nullptr;

  if (tid == 0) *sFlag = 0;

  // ---- inputs of my tokens (zero past the end) ---------------------------------
  const int c0 = (tid % CG) * 8, tq0 = (tid / CG) * TT, qg_ = lane / CG;
  const int t0 = n * CH;
  float kv[TT][8], qv[TT][8], ev[TT][8], gv[TT][8];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    const bool ok = t0 + tq0 + u < T;
    const size_t to = (size_t)min(t0 + tq0 + u, T - 1) * H;
    const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(kg + to * DK + c0);
    const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(qg + to * DK + c0);
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(g_seq + to * DK + c0);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(g_seq + to * DK + c0 + 4);
    f32x4 b0, b1;
    float bt = 0.f;
    if constexpr (erase_ch) {
      b0 = *reinterpret_cast<const f32x4*>(b_seq + to * DK + c0);
      b1 = *reinterpret_cast<const f32x4*>(b_seq + to * DK + c0 + 4);
    } else {
      bt = beta_seq[to];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kv[u][i] = ok ? (float)k8[i] : 0.f;
      qv[u][i] = ok ? (float)q8[i] : 0.f;
      gv[u][i] = ok ? (i < 4 ? g0[i] : g1[i - 4]) * LOG2E : 0.f;
      if constexpr (erase_ch) ev[u][i] = (i < 4 ? b0[i] : b1[i - 4]) * kv[u][i];
      else ev[u][i] = bt * __builtin_fmaf(lam, qv[u][i], kv[u][i]);
    }
  }
  __syncthreads();

  // ---- in-block prefix sums of the log-decay (base 2) ---------------------------
  // Hl = prefix over my TT tokens; Hsx = (sum at the block's first token) -
  // (sum over the token groups before mine): the decay of my token u relative
  // to the block start is dl = Hsx - Hl[u] >= 0.
  float Hl[TT][8], Hsx[8];
  {
    float excl[8], tot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < TT; ++u) {
        sum += gv[u][i];
        Hl[u][i] = sum;
      }
      tot[i] = sum;
      float x = sum;
#pragma unroll
      for (int d = CG; d < 64; d *= 2) {
        const float y = __shfl_up(x, d);
        x += lane >= d ? y : 0.f;
      }
      excl[i] = x - sum;
    }
    if (qg_ == 0) st8(sBt + w * DK + c0, Hl[0]);
    if (qg_ == 64 / CG - 1) {
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
    if (bad) *sFlag = 1;
  }
  __syncthreads();

  // ---- per-(block, channel) constants, base 2: P_J = G before block J,
  // G_sJ = P_J + Bt[J], G_C = P_4 ------------------------------------------------
  if (tid < DK) {
    const int c = tid;
    float P[5], gs[4];
    P[0] = 0.f;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      gs[J] = P[J] + sBt[J * DK + c];
      P[J + 1] = P[J] + sBt[(4 + J) * DK + c];
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      sEs[J * DK + c] = __builtin_amdgcn_exp2f(gs[J]);
      sF[J * DK + c] = __builtin_amdgcn_exp2f(P[4] - gs[J]);
    }
#pragma unroll
    for (int I = 1; I < 4; ++I)
#pragma unroll
      for (int J = 0; J < I; ++J) sD[(I * (I - 1) / 2 + J) * DK + c] = __builtin_amdgcn_exp2f(gs[I] - gs[J]);
    reinterpret_cast<float*>(rec + R::oGc)[c] = __builtin_amdgcn_exp2f(P[4]);
  }
  __syncthreads();

  // ---- bounded factors of my rows to LDS; E_bar, Q_gamma, K_tail rows out -----
  {
    const V8<float> es = ld8(sEs + w * DK + c0), fk = ld8(sF + w * DK + c0);
    const bool bad = *sFlag != 0;
    float lf[8];  // base-2 G_C - G_sw, for K_tail of a chunk past the window limit
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lf[i] = -sBt[w * DK + c0 + i];
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J >= w) lf[i] += sBt[(4 + J) * DK + c0 + i];
    }
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      const int t = tq0 + u;
      float kb[8], xe[8], xq[8], kt[8], eb[8], qgm[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float dl = Hsx[i] - Hl[u][i];  // >= 0
        const float ir = __builtin_amdgcn_exp2f(-dl);
        kb[i] = kv[u][i] * __builtin_amdgcn_exp2f(dl);
        xe[i] = ev[u][i] * ir;
        xq[i] = qv[u][i] * ir;
        kt[i] = kb[i] * fk[i];  // k exp(G_C - G) <= |k|
        eb[i] = xe[i] * es[i];
        qgm[i] = xq[i] * es[i];
      }
      if (bad) {
        // kb may have overflowed (the chunk takes the exact Gram): K_tail
        // from its own exponent, G_C - G = (G_C - G_sw) + dl
#pragma unroll
        for (int i = 0; i < 8; ++i) kt[i] = kv[u][i] * __builtin_amdgcn_exp2f(lf[i] + Hsx[i] - Hl[u][i]);
      }
      st8(sKb + t * SE + c0, kb);
      st8(sXe + t * SE + c0, xe);
      st8(sXq + t * SE + c0, xq);
      st8(reinterpret_cast<bf16*>(rec + R::oEb) + t * DK + c0, eb);
      st8(reinterpret_cast<bf16*>(rec + R::oQg) + t * DK + c0, qgm);
      st8(reinterpret_cast<bf16*>(rec + R::oKt) + t * DK + c0, kt);
    }
  }
  __syncthreads();

  // ---- T and A_qk tiles: wave w takes its diagonal tile and a share of the
  // six below the diagonal; A_qk goes straight out -------------------------------
  {
    bf16* aqk_out = reinterpret_cast<bf16*>(rec + R::oAqk);
    auto tiles = [&](auto tl) __attribute__((always_inline)) {
      using TL = decltype(tl);
      constexpr int NT = TL::n;
      f32x4 accT[NT], accA[NT], aqk[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) accT[t] = accA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (*sFlag == 0) {
        gram_bounded_tiles<DK, SE>(tl, sKb, sXe, sXq, sD, accT, accA, g, l16);
      } else {
        float* st = reinterpret_cast<float*>(smem + L::oKb) + w * (CH * 4 * SW);
        gram_exact_tiles<DK, SW, erase_ch>(tl, st, kg, qg, g_seq, b_seq, beta_seq, qmix, lam, n, T, H, accT, accA,
                                           lane, g, l16);
      }
      gram_mask_tiles<SC, TDS, TDB>(tl, accT, accA, aqk, sT, sTd, g, l16);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(aqk_out) +
                                   tri_lower_byte(16 * TL::I(t) + l16, 16 * TL::J(t) + 4 * g)) = cvt4(aqk[t]);
    };
    switch (w) {
      case 0: tiles(TileList<0, 0, 3, 0, 3, 1>{}); break;
      case 1: tiles(TileList<1, 1, 1, 0>{}); break;
      case 2: tiles(TileList<2, 2, 2, 0, 2, 1>{}); break;
      default: tiles(TileList<3, 3, 3, 2>{}); break;
    }
  }
  __syncthreads();
  // A's buffer (the xq rows, now read by no one) starts at zero above the
  // diagonal blocks
  for (int e = tid; e < CH * SC * 2 / 16; e += 256) reinterpret_cast<uint4*>(sA)[e] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  // ---- A = (I + T)^{-1}: waves 0 and 1 split its last level --------------------
  if (w == 0) solve_inverse<SC, TDS, TDB, 1>(sTd, sT, sA, g, l16);
  else if (w == 1) solve_inverse<SC, TDS, TDB, 2>(sTd, sT, sA, g, l16);
  __syncthreads();
  // the ten stored blocks of A (column-major)
  for (int q = tid; q < R::PIECES_A; q += 256) {
    const TriPiece pc = tri_upper_piece(q);
    reinterpret_cast<uint4*>(rec + R::oAcm)[q] = *reinterpret_cast<const uint4*>(sA + pc.row * SC + 8 * pc.col);
  }
}

// ---- pass 2 ------------------------------------------------------------------
template <int DK, int DVS>
struct RecLay {
  static constexpr int NCW = pipe_ncw<DVS>(), NB = DVS / (16 * NCW);
  static constexpr int SE = DK + 8, SKT = DK + 32, SC = CH + 8, SZ = DVS + 8, SO = CH + 8;
  static constexpr int szE = CH * SE * 2, szK = CH * SKT * 2, szA = CH * SC * 2, szZ = CH * SZ * 2;
  // two buffers of each, by chunk parity
  static constexpr int oEb = 0, oQg = 2 * szE, oKt = 4 * szE, oAcm = oKt + 2 * szK, oAqk = oAcm + 2 * szA;
  static constexpr int oZ = oAqk + 2 * szA, oGc = oZ + 2 * szZ;
  static constexpr int oStage = oGc + 2 * DK * 4;  // O staging, [value column][token] per consumer wave
  static constexpr int TOTAL = oStage + DVS * SO * 2;
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
  static_assert(oQg % 16 == 0 && oKt % 16 == 0 && oAcm % 16 == 0 && oAqk % 16 == 0 && oZ % 16 == 0 &&
                    oGc % 16 == 0 && oStage % 16 == 0,
                "alignment");
};

template <int DK, int DVS, int GM>
__global__ __launch_bounds__(64 * (pipe_ncw<DVS>() + 4)) void chan_rec_kernel(ChunkParams p,
                                                                              const char* __restrict__ ws) {
  static_assert(DK == 128, "record layout: 16 pieces of 16 bytes per row");
  using L = RecLay<DK, DVS>;
  using R = SplitRec<DK>;
  constexpr int NCW = L::NCW, NB = L::NB;
  constexpr int SE = L::SE, SKT = L::SKT, SC = L::SC, SZ = L::SZ, SO = L::SO;
  constexpr int NKS = DK / 32;
  constexpr bool write_ch = Gates<GM>::WRITE_CH;

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  // workgroup -> (batch, head, value slice); the slices of a head run on one
  // XCD and share its L2, where they find each other's records
  int wid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int NS = p.nslices;
  const int bh = wid / NS, slice = wid - bh * NS;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H, DV = p.DV;
  const int vbase = slice * DVS;
  const int nchunks = (T + CH - 1) / CH;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const char* recs = ws + (size_t)bh * nchunks * R::BYTES;

  // the blocks above the diagonal of A and A_qk (not in the record) stay zero
  static_assert(L::oAqk == L::oAcm + 2 * L::szA, "A and A_qk buffers adjacent");
  for (int e = tid; e < 4 * L::szA / 16; e += 64 * (NCW + 4))
    reinterpret_cast<uint4*>(smem + L::oAcm)[e] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();

  if (wave < NCW) {
    // =================== consumers (as in chan_kernel.hpp) ====================
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
    bf16* stage = reinterpret_cast<bf16*>(smem + L::oStage) + wave * (16 * NB) * SO;

    // step n applies chunk n - 1 (the loaders bring chunk n meanwhile)
    for (int n = 0; n <= nchunks; ++n) {
      if (n > 0) {
        const int c = n - 1, buf = c & 1;
        const bf16* sEb = reinterpret_cast<const bf16*>(smem + L::oEb + buf * L::szE);
        const bf16* sQg = reinterpret_cast<const bf16*>(smem + L::oQg + buf * L::szE);
        const bf16* sKt = reinterpret_cast<const bf16*>(smem + L::oKt + buf * L::szK);
        const bf16* sAcm = reinterpret_cast<const bf16*>(smem + L::oAcm + buf * L::szA);
        const bf16* sAqk = reinterpret_cast<const bf16*>(smem + L::oAqk + buf * L::szA);
        const bf16* sZ = reinterpret_cast<const bf16*>(smem + L::oZ + buf * L::szZ);
        const float* gC = reinterpret_cast<const float*>(smem + L::oGc) + buf * DK;

        // The three phases of a chunk run back to back in this wave, so each
        // requests the next one's LDS fragments before its own products:
        // A (transposing reads) and A_qk rows for W and O, K_tail^T and
        // gamma_C for the state update.
        auto afrag = [&](int pp, int h, int m2) __attribute__((always_inline)) {
          const int col = 32 * pp + 8 * (l16 & 3) + 4 * h;
          return cat8(lds_tr4(sAcm + (32 * m2 + 4 * g + (l16 >> 2)) * SC + col),
                      lds_tr4(sAcm + (32 * m2 + 16 + 4 * g + (l16 >> 2)) * SC + col));
        };
        bf16x8 Af[2][2][2], Aq[4][2], Kt[2 * NKS][2];
        f32x4 Gc[2 * NKS];

        // E_bar S and Q_gamma S
        f32x4 ES[4][NB], QS[4][NB];
        {
          bf16x8 Sb[NKS][NB];
#pragma unroll
          for (int m = 0; m < NKS; ++m)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Sb[m][nb] = cat8(cvt4(S[2 * m][nb]), cvt4(S[2 * m + 1][nb]));
          // fragments of row block I + 2 are requested while block I multiplies
          bf16x8 ef[3][NKS], qf[3][NKS];
          auto load_eq = [&](int I, int slot) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
              ef[slot][m] = *reinterpret_cast<const bf16x8*>(sEb + (16 * I + l16) * SE + 32 * m + 8 * g);
              qf[slot][m] = *reinterpret_cast<const bf16x8*>(sQg + (16 * I + l16) * SE + 32 * m + 8 * g);
            }
          };
          load_eq(0, 0);
          load_eq(1, 1);
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            if (I + 2 < 4) load_eq(I + 2, (I + 2) % 3);
            if (I == 2) {
#pragma unroll
              for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                  for (int m2 = 0; m2 <= pp; ++m2) Af[pp][h][m2] = afrag(pp, h, m2);
#pragma unroll
              for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int pp = 0; pp <= J / 2; ++pp)
                  Aq[J][pp] = *reinterpret_cast<const bf16x8*>(sAqk + (16 * J + l16) * SC + 32 * pp + 8 * g);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              ES[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
              QS[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int m = 0; m < NKS; ++m) {
                ES[I][nb] = mma32(ef[I % 3][m], Sb[m][nb], ES[I][nb]);
                QS[I][nb] = mma32(qf[I % 3][m], Sb[m][nb], QS[I][nb]);
              }
            }
          }
        }

        // W = A (Z - E_bar S), O = Q_gamma S + A_qk W
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
              for (int m2 = 0; m2 <= pp; ++m2)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[nb] = mma32(Af[pp][h][m2], Rb[m2][nb], acc[nb]);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) Wt[2 * pp + h][nb] = acc[nb];
            }
          // the state update's fragments, requested behind W's products
#pragma unroll
          for (int j = 0; j < 2 * NKS; ++j) {
            const int col = 32 * (j >> 1) + 8 * (l16 & 3) + 4 * (j & 1);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
              Kt[j][pp] = cat8(lds_tr4(sKt + (32 * pp + 8 * g + (l16 >> 2)) * SKT + col),
                               lds_tr4(sKt + (32 * pp + 8 * g + 4 + (l16 >> 2)) * SKT + col));
            // rows of state tile j: channels 32 (j/2) + 8 g + 4 (j%2) + r
            Gc[j] = *reinterpret_cast<const f32x4*>(gC + 32 * (j >> 1) + 8 * g + 4 * (j & 1));
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
            for (int pp = 0; pp <= I / 2; ++pp)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) Oh[I][nb] = mma32(Aq[I][pp], Wb[pp][nb], Oh[I][nb]);
          }
        }

        // S = Diag(gamma_C) S + K_tail^T W; outputs
        {
          bf16x8 Wtb[2][NB];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Wtb[pp][nb] = cat8(cvt4(Wt[2 * pp][nb]), cvt4(Wt[2 * pp + 1][nb]));
#pragma unroll
          for (int j = 0; j < 2 * NKS; ++j) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              f32x4 acc = S[j][nb] * Gc[j];
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) acc = mma32(Kt[j][pp], Wtb[pp][nb], acc);
              S[j][nb] = acc;
            }
          }
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
            const int t = c * CH + 16 * g + l16;
            if (t < T) *reinterpret_cast<bf16x8*>(og + t * H * DV + cw0 + 8 * k) = v;
          }
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
    // =================== loaders ===============================================
    // Record pieces of 16 bytes: lane lt copies piece lt + 256 k of E_bar,
    // Q_gamma and K_tail (k < 4 each; 1,024 pieces per region) and piece lt
    // of the stored A and A_qk triangles (320 pieces each); the remaining 64
    // pieces of A go to loader wave 1, those of A_qk to wave 2 and gamma_C
    // (32 pieces) to wave 0, so that wave 3, which shares its SIMD with the
    // first consumer wave, issues the fewest loads.  Z = gate * v of the slice is formed from its
    // own loads, ZC columns of one token per lane, so that every loader lane
    // takes an equal share of it.
    const int lt = tid - 64 * NCW;
    const int lw = wave - NCW, l64 = lt & 63;  // loader wave (uniform), lane in it
    constexpr int qA = R::oAcm / 16, qAqk = R::oAqk / 16, qGc = R::oGc / 16;  // region starts, in pieces
    // LDS destinations (bytes, buffer 0) of the triangle pieces
    const TriPiece pa = tri_upper_piece(lt), pq = tri_lower_piece(lt);
    const int dA = L::oAcm + pa.row * SC * 2 + pa.col * 16, dAq = L::oAqk + pq.row * SC * 2 + pq.col * 16;
    int xsrc = 0, xdst = 0, xstride = 0;  // the extra piece of waves 1-3
    if (lw == 1) {
      const TriPiece t = tri_upper_piece(256 + l64);
      xsrc = qA + 256 + l64, xdst = L::oAcm + t.row * SC * 2 + t.col * 16, xstride = L::szA;
    } else if (lw == 2) {
      const TriPiece t = tri_lower_piece(256 + l64);
      xsrc = qAqk + 256 + l64, xdst = L::oAqk + t.row * SC * 2 + t.col * 16, xstride = L::szA;
    } else if (lw == 0) {
      xsrc = qGc + min(l64, 31), xdst = L::oGc + l64 * 16, xstride = DK * 4;
    }
    const bool xwrite = lw == 1 || lw == 2 || (lw == 0 && l64 < 32);
    constexpr int ZC = DVS / 4;                 // Z columns per lane (64 DVS values over 256 lanes)
    constexpr int VG = DVS / ZC;                // lanes per v row
    const int tz = lt / VG, vv0 = (lt % VG) * ZC;
    typedef bf16 bfz __attribute__((ext_vector_type(ZC)));
    const bf16* vg = reinterpret_cast<const bf16*>(p.v) + seq0 * DV + vbase;
    const float* beta_seq = p.beta ? p.beta + seq0 : nullptr;
    const float* w_seq = write_ch ? p.w + seq0 * DV + vbase : nullptr;
    // (clang vector elements: arrays of HIP's uint4 struct stay in scratch
    // memory instead of registers)
    u32x4 rE[4], rQ[4], rK[4], rAc, rAq, rX = {};
    bfz rv = {};
    f32x4 rw[write_ch ? ZC / 4 : 1] = {};
    float rvb = 0.f;
    // Loads are unconditional, at chunk indices clamped to the last one.
#define GDR_SPLIT_LOAD(nl)                                                                  \
    {                                                                                       \
      const int n_ = (nl);                                                                  \
      const u32x4* rec0 = reinterpret_cast<const u32x4*>(recs + (size_t)n_ * R::BYTES);     \
      const u32x4* rec = rec0 + lt;                                                         \
      _Pragma("unroll") for (int k = 0; k < 4; ++k) {                                       \
        rE[k] = rec[256 * k];                                                               \
        rQ[k] = rec[1024 + 256 * k];                                                        \
        rK[k] = rec[2048 + 256 * k];                                                        \
      }                                                                                     \
      rAc = rec[qA];                                                                        \
      rAq = rec[qAqk];                                                                      \
      if (lw != 3) rX = rec0[xsrc];                                                         \
      {                                                                                     \
        const unsigned r = (unsigned)(min(n_ * CH + tz, T - 1) - n_ * CH) * H;              \
        rv = *reinterpret_cast<const bfz*>(vg + (size_t)n_ * CH * H * DV + r * DV + vv0);   \
        if constexpr (write_ch) {                                                           \
          const float* wc = w_seq + (size_t)n_ * CH * H * DV + r * DV + vv0;               \
          _Pragma("unroll") for (int i = 0; i < ZC / 4; ++i)                               \
            rw[i] = *reinterpret_cast<const f32x4*>(wc + 4 * i);                            \
        } else {                                                                            \
          rvb = beta_seq[(size_t)n_ * CH * H + r];                                          \
        }                                                                                   \
      }                                                                                     \
    }
    if (nchunks > 0) GDR_SPLIT_LOAD(0)
    for (int n = 0; n <= nchunks; ++n) {
      // (at n = nchunks the last chunk is written again, into the buffer
      // that no one reads any more)
      if (nchunks > 0) {
        const int nw = min(n, nchunks - 1), buf = n & 1;
        // rows of 16 pieces (E_bar, Q_gamma, K_tail), then the triangles
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = lt + 256 * k, row = q >> 4, col = q & 15;
          *reinterpret_cast<u32x4*>(smem + L::oEb + buf * L::szE + row * SE * 2 + col * 16) = rE[k];
          *reinterpret_cast<u32x4*>(smem + L::oQg + buf * L::szE + row * SE * 2 + col * 16) = rQ[k];
          *reinterpret_cast<u32x4*>(smem + L::oKt + buf * L::szK + row * SKT * 2 + col * 16) = rK[k];
        }
        *reinterpret_cast<u32x4*>(smem + dA + buf * L::szA) = rAc;
        *reinterpret_cast<u32x4*>(smem + dAq + buf * L::szA) = rAq;
        if (xwrite) *reinterpret_cast<u32x4*>(smem + xdst + buf * xstride) = rX;
        {
          const bool ok = nw * CH + tz < T;
          float z[ZC];
#pragma unroll
          for (int e = 0; e < ZC; ++e) {
            float gate;
            if constexpr (write_ch) gate = rw[e / 4][e % 4];
            else gate = rvb;
            z[e] = ok ? gate * (float)rv[e] : 0.f;
          }
          bf16* zd = reinterpret_cast<bf16*>(smem + L::oZ + buf * L::szZ) + tz * SZ + vv0;
          if constexpr (ZC == 8) st8(zd, z);
          else *reinterpret_cast<bf16x4*>(zd) = cvt4(f32x4{z[0], z[1], z[2], z[3]});
        }
        GDR_SPLIT_LOAD(min(n + 1, nchunks - 1))
      }
      __syncthreads();
    }
#undef GDR_SPLIT_LOAD
  }
}

template <int DK>
constexpr int split_rec_bytes() {
  return SplitRec<DK>::BYTES;
}

}  // namespace gdr
