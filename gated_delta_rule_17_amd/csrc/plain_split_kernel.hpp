// Two-pass form of the plain fp32 chunk kernel (plain_kernel.hpp): the same
// chunk WY form with absorbed decay ("Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention", key design 2), all arithmetic fp32, with the
// state-independent work of a chunk done once per (batch, head, chunk)
// instead of once per value slice:
//
//   pass 1  plain_prep_kernel, one workgroup per chunk: the gates, the
//           chunk-local prefix sums G of the log-decay, the factor rows
//             E_bar = e (.) exp(G),  Q_gamma = q (.) exp(G),
//             K_tail = k (.) exp(G_C - G),  gamma_C = exp(G_C)
//           the Gram matrices
//             T[i][j]   = sum_c e_i[c] k_j[c] exp(G_i[c] - G_j[c])   j <  i
//             Aqk[i][j] = sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])   j <= i
//           (zeros elsewhere) and the inverse A = (I + T)^{-1} (diagonal
//           16 x 16 blocks by forward substitution, then the blocks below
//           them block row by block row), written to the record arrays of a
//           BwdWs: A in the place of T, or T itself under the
//           per-value-channel beta, whose systems differ per column.
//   pass 2  plain_rec_kernel, one workgroup per (batch, head, 16-column value
//           slice), chunks in order, the state slice in LDS:
//             ES = E_bar S, QS = Q_gamma S,
//             W = A (Z - ES), or under the per-value-channel beta the
//               solution of (I + M (.) T) W = Z - M (.) ES by forward
//               substitution, column by column,
//             O = QS + Aqk W,  S <- Diag(gamma_C) S + K_tail^T W.
//
// Every exponent is <= 0 (G is non-increasing along the chunk), so no factor
// leaves the fp32 range.  Under a scalar decay (or none) exp(G_i - G_j) is
// the same for every channel and multiplies the channel sums; under a decay
// per key channel it is formed per term.  The erase direction e is
// beta (k + lambda q) (lambda = 0 without the Q-Delta mix; per head or per
// token), b (.) k for the per-channel erase gate, or k under the
// per-value-channel beta, whose strength M then sits in the substitution.
//
// The record pass of the backward (bwd_kernel.hpp) is pass 1 followed by
// pass 2 in record mode (REC), which writes, per chunk, the entering state
// and W of its slice instead of o.
#pragma once

#include "bwd_params.hpp"
#include "common.hpp"
#include "plain_kernel.hpp"

namespace gdr {

// ---- split precision ------------------------------------------------------
// Products on the bf16 matrix cores with near-fp32 operands: each fp32
// operand x is held as hi = bf16(x) and lo = bf16(x - hi), and X Y is formed
// as Xhi Yhi + Xhi Ylo + Xlo Yhi (v_mfma_f32_16x16x32_bf16, fp32
// accumulation; the dropped Xlo Ylo and the roundings of lo leave about 16
// bits of each operand).  In a 32-wide k-step m, lane group g = l / 16 takes
// the k indices 32 m + 4 g + e and 32 m + 16 + 4 g + e (e < 4), which is
// where a lane's accumulators hold them in the tiles 2m and 2m + 1, so
// accumulator tiles serve as B operands once split (split_b).  Operands in
// LDS are rows stored with their k index in that order: kpos(x) is the
// position of k index x in such a row.
__device__ __forceinline__ constexpr int kpos(int x) {
  return (x & ~31) + 8 * ((x & 15) >> 2) + 4 * ((x >> 4) & 1) + (x & 3);
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f32x4 fl4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }
__device__ __forceinline__ bf16x8 join8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// four consecutive values (k index x, a multiple of 4) of row r of a split
// operand with row stride S: hi to arr, lo to arr + half
template <int S>
__device__ __forceinline__ void put_split(bf16* arr, int half, int r, int x, f32x4 v) {
  const bf16x4 hi = bf4(v);
  bf16* d = arr + r * S + kpos(x);
  *reinterpret_cast<bf16x4*>(d) = hi;
  *reinterpret_cast<bf16x4*>(d + half) = bf4(v - fl4(hi));
}
// B operand of k-step m from accumulator tiles t0 (k slots e < 4) and t1
struct SplitB {
  bf16x8 hi, lo;
};
__device__ __forceinline__ SplitB split_b(f32x4 t0, f32x4 t1) {
  const bf16x4 h0 = bf4(t0), h1 = bf4(t1);
  return SplitB{join8(h0, h1), join8(bf4(t0 - fl4(h0)), bf4(t1 - fl4(h1)))};
}
// acc += A B in split precision, A from its two halves at a (lo at a + half)
__device__ __forceinline__ f32x4 mma_split(const bf16* a, int half, const SplitB& b, f32x4 acc) {
  const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(a), alo = *reinterpret_cast<const bf16x8*>(a + half);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b.lo, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b.hi, acc, 0, 0, 0);
}
// a fragment of a split operand stored in LDS (hi at a, lo at a + half)
__device__ __forceinline__ SplitB lds_split(const bf16* a, int half) {
  return SplitB{*reinterpret_cast<const bf16x8*>(a), *reinterpret_cast<const bf16x8*>(a + half)};
}
// acc += A B in split precision, both operands as fragments
__device__ __forceinline__ f32x4 mma_split(const SplitB& a, const SplitB& b, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
}

// ---- pass 1 -----------------------------------------------------------------
// Channels are processed in halves of 64, 74 KB of LDS (two workgroups per
// CU); the next half's loads are in flight during a half's Gram sums.  Under
// a scalar decay (or none) the Gram sums are MFMA tiles in split precision
// (k, e, q of the half staged as bf16 hi and lo rows in kpos order, both
// operands 16-byte reads of rows, two 32-wide k-steps per half): wave w owns
// the (I, J) tile pairs w, w + 4, w + 8 of the ten on or below the diagonal.
// Under a decay per key channel every term carries its own exponential and
// the sums run on the vector ALUs from [64][68] fp32 arrays of k, e, q and
// the prefix sums G of the half, 4 x 4 (i, j) blocks per thread.
struct PlainPrepLay {
  static constexpr int CHH = 64;       // channels per half
  static constexpr int HP = CHH + 4;   // row stride (floats): 16-byte rows
  static constexpr int oK = 0, oX = oK + CH * HP, oQ = oX + CH * HP, oG = oQ + CH * HP;
  static constexpr int oGs = oG + CH * HP;  // [64] scalar-decay prefix sums
  static constexpr int oPart = oGs + CH;    // [16][64] sums of the log-decay over 4-row groups
  static constexpr int TOTAL = oPart + 16 * CHH;
  static_assert(2 * TOTAL * 4 <= 160 * 1024, "two workgroups per CU");
  // under a scalar decay (or none): k, e, q of the half split into bf16 hi
  // and lo halves ([64][SE] each, kpos order), over the fp32 arrays
  static constexpr int SE = CHH + 8, HS = CH * SE;  // row stride, elements per half
  static constexpr int oKs = 0, oXs = 2 * HS, oQs = 4 * HS;
  static_assert(6 * HS * 2 <= oGs * 4 && (SE * 2) % 16 == 0, "split arrays below the scalars");
};

// A = (I + T)^{-1} from T (sT: dense [64][HP] fp32, zero on and above the
// diagonal) into sAi, sP as scratch; then A to recA, the chunk's [64][64]
// record (zero above the diagonal).  Every thread of the workgroup calls
// it, after a barrier that follows the writes of sT.
template <int HP>
__device__ __forceinline__ void prep_inverse(const float* sT, float* sAi, float* sP, float* recA, int tid) {
  // ---- A = (I + T)^{-1} ------------------------------------------------------
  // level 0: the diagonal blocks (I + T_bb)^{-1}; thread 16 b + l solves for
  // column l of block b (x = e_l, then x_i -= sum_{m < i} T_im x_m)
  if (tid < CH) {
    const int r0 = 16 * (tid >> 4), l = tid & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = i == l ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = __builtin_fmaf(sT[(r0 + i) * HP + r0 + m], x[m], s);
      x[i] -= s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sAi[(r0 + i) * HP + r0 + l] = x[i];
  }
  __syncthreads();
  // levels s = 1, 2, 3: the blocks (I, J) with I - J = s,
  //   A_IJ = -A_II sum_{K = J}^{I - 1} T_IK A_KJ
  // (every A_KJ on the right lies closer to the diagonal)
  // (thread tid: element (i, j) = (tid / 16, tid % 16) of each block)
  const int bi = tid >> 4, bj = tid & 15;
  auto level = [&](auto slc) __attribute__((always_inline)) {
    constexpr int sl = decltype(slc)::value;
#pragma unroll
    for (int J = 0; J + sl < 4; ++J) {
      const int I = J + sl;
      float acc = 0.f;
#pragma unroll
      for (int kk = 16 * J; kk < 16 * I; ++kk)
        acc = __builtin_fmaf(sT[(16 * I + bi) * HP + kk], sAi[kk * HP + 16 * J + bj], acc);
      sP[(16 * J + bi) * HP + bj] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int J = 0; J + sl < 4; ++J) {
      const int I = J + sl;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc = __builtin_fmaf(sAi[(16 * I + bi) * HP + 16 * I + m], sP[(16 * J + m) * HP + bj], acc);
      sAi[(16 * I + bi) * HP + 16 * J + bj] = -acc;
    }
    __syncthreads();
  };
  level(IC<1>{});
  level(IC<2>{});
  level(IC<3>{});
  // A to the record in the place of T (zero above the diagonal)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + NTHR * u, i = e >> 4, j4 = (e & 15) * 4;
    f32x4 av;
#pragma unroll
    for (int b = 0; b < 4; ++b) av[b] = j4 + b <= i ? sAi[i * HP + j4 + b] : 0.f;
    *reinterpret_cast<f32x4*>(recA + i * CH + j4) = av;
  }
}

// factors = 0: the factor rows E_bar, Q_gamma, K_tail and gamma_C are not
// written (the passes that read them form them from the inputs: a scalar
// decay or none, see sd_rows).
template <class IO, int DK>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void plain_prep_kernel(ChunkParams p, BwdWs ws, int factors) {
  using L = PlainPrepLay;
  constexpr int HP = L::HP, CHH = L::CHH, NH = DK / CHH;
  static_assert(DK % CHH == 0, "whole halves");
  __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
  float* sK = lds + L::oK;
  float* sX = lds + L::oX;
  float* sQ = lds + L::oQ;
  float* sG = lds + L::oG;
  float* sGs = lds + L::oGs;
  float* sPart = lds + L::oPart;
  bf16* sp = reinterpret_cast<bf16*>(lds);
  constexpr int SE = L::SE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, H = p.H, N = (T + CH - 1) / CH;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int bb = bh / H, hh = bh - bb * H;
  const int t0 = n * CH;
  const size_t ch = blockIdx.x;  // record index (batch * H + head) * N + chunk
  const size_t seq0 = (size_t)bb * T * H + hh;
  const int decay = p.decay, erase = p.erase, qmix = p.qmix;
  const IO* qg = reinterpret_cast<const IO*>(p.q);
  const IO* kg = reinterpret_cast<const IO*>(p.k);

  // scalar decay: prefix sums of the chunk's per-token log-decay (zero past T)
  if (wave == 0) {
    const int t = t0 + lane;
    const float g = (decay == 1 && t < T) ? p.g[seq0 + (size_t)t * H] : 0.f;
    sGs[lane] = wave_incl_scan(g);
  }

  // elementwise layout: thread = rows 4 rg .. 4 rg + 3 x channels c4 .. c4 + 3
  // of the half (16 threads cover a row's 64 channels: coalesced rows)
  const int rg = tid >> 4, c4 = (tid & 15) * 4;
  // Gram layout: 4 x 4 blocks (ib, jb) of (i, j), blocks with jb <= ib
  const int ib = tid >> 4, jb = tid & 15;
  float accT[4][4], accA[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) accT[a][b] = accA[a][b] = 0.f;
  // matrix-core layout: tile pair pr = wave + 4 t (t < 3, pr < 10) of the
  // ten (I >= J) in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ..
  const int g = lane >> 4, l16 = lane & 15;
  auto tile_I = [](int pr) { return pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3; };
  auto tile_J = [](int pr) { return pr - (pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 3 : 6); };
  f32x4 mT[3], mA[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) mT[t] = mA[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- loads of a half: every load of the thread, at token indices clamped
  // to T - 1, masked at use
  f32x4 rk[4], rq[4], rgc[4], rb[4];
  float rbeta[4], rlam[4];
  auto load_half = [&](int cb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * rg + u;
      const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
      rk[u] = ldf4(kg + tok * DK + cb + c4);
      rq[u] = ldf4(qg + tok * DK + cb + c4);
      if (decay == 2) rgc[u] = *reinterpret_cast<const f32x4*>(p.g + tok * DK + cb + c4);
      if (erase == 1) rb[u] = *reinterpret_cast<const f32x4*>(p.b + tok * DK + cb + c4);
      rbeta[u] = erase == 0 ? p.beta[tok] : 0.f;
      rlam[u] = qmix == 2 ? p.lam[tok] : (qmix ? p.lam[hh] : 0.f);
    }
  };
  load_half(0);

#pragma unroll
  for (int half = 0; half < NH; ++half) {
    const int cb = half * CHH;  // first channel of the half
    // (sGs ready, sPart free; after the first half: its Gram reads are done)
    __syncthreads();
    // ---- prefix sums of the log-decay per channel: within the thread's four
    // rows, then over the 4-row groups through sPart
    float G[4][4];  // [row u][channel i]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float run = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = t0 + 4 * rg + u < T;
        run += (decay == 2 && ok) ? rgc[u][i] : 0.f;
        G[u][i] = run;
      }
    }
    float GC[4];
    if (decay == 2) {
      *reinterpret_cast<f32x4*>(sPart + rg * CHH + c4) = f32x4{G[3][0], G[3][1], G[3][2], G[3][3]};
      __syncthreads();
      f32x4 excl = {0.f, 0.f, 0.f, 0.f}, tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const f32x4 s = *reinterpret_cast<const f32x4*>(sPart + q * CHH + c4);
        if (q < rg) excl += s;
        tot += s;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u) G[u][i] += excl[i];
        GC[i] = tot[i];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) G[u][i] = sGs[4 * rg + u];
#pragma unroll
      for (int i = 0; i < 4; ++i) GC[i] = sGs[CH - 1];
    }
    // ---- erase directions, factor rows to the record, operands to LDS ------
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 4 * rg + u;
      const bool ok = t0 + r < T;
      f32x4 kv, qv, ev, eb, qgm, kt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kv[i] = ok ? rk[u][i] : 0.f;
        qv[i] = ok ? rq[u][i] : 0.f;
        if (erase == 1) ev[i] = rb[u][i] * kv[i];
        else if (erase == 2) ev[i] = kv[i];
        else ev[i] = rbeta[u] * __builtin_fmaf(rlam[u], qv[i], kv[i]);
        if (!ok) ev[i] = 0.f;
        const float gam = fexp(G[u][i]);
        eb[i] = ev[i] * gam;
        qgm[i] = qv[i] * gam;
        kt[i] = kv[i] * fexp(GC[i] - G[u][i]);
      }
      const size_t ro = (ch * CH + r) * DK + cb + c4;
      if (factors) {
        *reinterpret_cast<f32x4*>(ws.Eb + ro) = eb;
        *reinterpret_cast<f32x4*>(ws.Qg + ro) = qgm;
        *reinterpret_cast<f32x4*>(ws.Kt + ro) = kt;
      }
      if (decay == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sK[r * HP + c4 + i] = kv[i];
          sX[r * HP + c4 + i] = ev[i];
          sQ[r * HP + c4 + i] = qv[i];
          sG[r * HP + c4 + i] = G[u][i];
        }
      } else {
        put_split<SE>(sp + L::oKs, L::HS, r, c4, kv);
        put_split<SE>(sp + L::oXs, L::HS, r, c4, ev);
        put_split<SE>(sp + L::oQs, L::HS, r, c4, qv);
      }
    }
    if (rg == 0 && factors) {
      *reinterpret_cast<f32x4*>(ws.gC + ch * DK + cb + c4) =
          f32x4{fexp(GC[0]), fexp(GC[1]), fexp(GC[2]), fexp(GC[3])};
    }
    // the next half's loads, in flight during this half's Gram sums
    if (half + 1 < NH) load_half(cb + CHH);
    __syncthreads();
    // ---- Gram sums over the half's channels ----------------------------------
    if (decay != 2) {
      // split precision, two 32-wide k-steps per half
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int pr = wave + 4 * t;
        if (pr >= 10) continue;  // wave-uniform
        const int I = tile_I(pr), J = tile_J(pr);
#pragma unroll
        for (int m = 0; m < CHH / 32; ++m) {
          const bf16* base = sp + l16 * SE + 32 * m + 8 * g;
          const SplitB bk = lds_split(base + L::oKs + 16 * J * SE, L::HS);
          const SplitB ax = lds_split(base + L::oXs + 16 * I * SE, L::HS);
          const SplitB aq = lds_split(base + L::oQs + 16 * I * SE, L::HS);
          mT[t] = mma_split(ax, bk, mT[t]);
          mA[t] = mma_split(aq, bk, mA[t]);
        }
      }
    } else if (jb <= ib) {
      for (int c = 0; c < CHH; ++c) {
        float xi[4], qi[4], kj[4], gi[4], gj[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int i = 4 * ib + a, j = 4 * jb + a;
          xi[a] = sX[i * HP + c];
          qi[a] = sQ[i * HP + c];
          kj[a] = sK[j * HP + c];
          gi[a] = sG[i * HP + c];
          gj[a] = sG[j * HP + c];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            // exponent clamped at 0: entries above the diagonal are discarded
            const float kd = kj[b] * fexp(fminf(gi[a] - gj[b], 0.f));
            accT[a][b] = __builtin_fmaf(xi[a], kd, accT[a][b]);
            accA[a][b] = __builtin_fmaf(qi[a], kd, accA[a][b]);
          }
      }
    }
  }
  // ---- Aqk to the record, T to LDS (dense [64][64], zeros above the masks) -
  __syncthreads();  // every Gram read of the operand arrays is done
  float* sT = lds + L::oK;   // [64][HP] T
  float* sAi = lds + L::oX;  // [64][HP] A = (I + T)^{-1}
  float* sP = lds + L::oQ;   // [48][HP] block products of the inverse's levels
  // (under the per-value-channel beta every column has its own system: T
  // itself goes to the record)
  if (decay == 2) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = 4 * ib + a;
      f32x4 tv, av;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = 4 * jb + b;
        tv[b] = (jb <= ib && j < i) ? accT[a][b] : 0.f;
        av[b] = (jb <= ib && j <= i) ? accA[a][b] : 0.f;
        sT[i * HP + j] = tv[b];
      }
      *reinterpret_cast<f32x4*>(ws.A + ch * CH * CH + i * CH + 4 * jb) = av;
      if (erase == 2) *reinterpret_cast<f32x4*>(ws.T + ch * CH * CH + i * CH + 4 * jb) = tv;
    }
  } else {
    // the tiles on and below the diagonal, times the common factor
    // exp(G_i - G_j) of the channels; lane: rows 16 I + 4 g + r, column 16 J + l16
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int pr = wave + 4 * t;
      if (pr >= 10) continue;
      const int I = tile_I(pr), J = tile_J(pr), j = 16 * J + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        const float d = fexp(fminf(sGs[i] - sGs[j], 0.f));
        const float tv = j < i ? mT[t][r] * d : 0.f, av = j <= i ? mA[t][r] * d : 0.f;
        sT[i * HP + j] = tv;
        ws.A[ch * CH * CH + i * CH + j] = av;
        if (erase == 2) ws.T[ch * CH * CH + i * CH + j] = tv;
      }
    }
    // the six tiles above the diagonal are zero in the record
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int u = wave + 4 * t;
      if (u >= 6) continue;
      const int I = u < 3 ? 0 : u < 5 ? 1 : 2, J = u < 3 ? u + 1 : u < 5 ? u - 1 : 3, j = 16 * J + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        ws.A[ch * CH * CH + i * CH + j] = 0.f;
        if (erase == 2) ws.T[ch * CH * CH + i * CH + j] = 0.f;
      }
    }
  }
  if (erase == 2) return;
  __syncthreads();
  prep_inverse<HP>(sT, sAi, sP, ws.T + ch * CH * CH, tid);
}

// ---- pass 1 with bf16 inputs under a scalar decay (or none) ------------------
// With bf16 k and q and the erase direction e = beta (k + lambda q), the Gram
// sums split into products of the raw inputs, exact on the bf16 matrix cores
// (fp32 accumulation), with the per-token scalars applied to the sums:
//   T[i][j]   = beta_i ((K K^T)[i][j] + lambda_i (Q K^T)[i][j]) exp(G_i - G_j)   j <  i
//   Aqk[i][j] = (Q K^T)[i][j] exp(G_i - G_j)                                     j <= i
// The rows are staged once as they arrive (no halves, no conversions); the
// inverse then takes their place.  48 KB of LDS: three workgroups per CU.
// The factor rows are not written (the passes that read them form them from
// the inputs).
template <int DK>
struct PlainPrepExactLay {
  static constexpr int SR = DK + 8;  // bf16 row stride: 16-row fragment reads in distinct banks
  static constexpr int HP = CH + 4;  // the inverse's fp32 arrays
  static constexpr int oRows = 0;    // k rows, then q rows: [64][SR] bf16 each (floats: CH * SR)
  static constexpr int oT = 0, oAi = oT + CH * HP, oP = oAi + CH * HP;  // [64][HP], [64][HP], [48][HP]
  static constexpr int END = (oP + 48 * HP) > CH * SR ? (oP + 48 * HP) : CH * SR;
  static constexpr int oGs = END, oBeta = oGs + CH, oLam = oBeta + CH;
  static constexpr int TOTAL = oLam + CH;
  static_assert(3 * TOTAL * 4 <= 160 * 1024, "three workgroups per CU");
  static_assert((SR * 2) % 16 == 0, "16-byte rows");
};

template <int DK>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(3, 3)))
void plain_prep_exact_kernel(ChunkParams p, BwdWs ws) {
  using L = PlainPrepExactLay<DK>;
  constexpr int SR = L::SR, HP = L::HP;
  __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
  bf16* sKr = reinterpret_cast<bf16*>(lds + L::oRows);
  bf16* sQr = sKr + CH * SR;
  float *sT = lds + L::oT, *sAi = lds + L::oAi, *sP = lds + L::oP;
  float *sGs = lds + L::oGs, *sBeta = lds + L::oBeta, *sLam = lds + L::oLam;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, H = p.H, N = (T + CH - 1) / CH;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int bb = bh / H, hh = bh - bb * H;
  const int t0 = n * CH;
  const size_t ch = blockIdx.x;  // record index (batch * H + head) * N + chunk
  const size_t seq0 = (size_t)bb * T * H + hh;
  const bf16* kg = reinterpret_cast<const bf16*>(p.k);
  const bf16* qg = reinterpret_cast<const bf16*>(p.q);

  // ---- rows of k and q (zero past T), every load of the thread first
  constexpr int RPT = CH * DK / 8 / NTHR;  // 16-byte pieces per thread and array
  bf16x8 rk[RPT], rq[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int e = tid + NTHR * u, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
    const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
    rk[u] = *reinterpret_cast<const bf16x8*>(kg + tok * DK + c8);
    rq[u] = *reinterpret_cast<const bf16x8*>(qg + tok * DK + c8);
  }
  // wave 0: prefix sums of the log-decay; wave 1: beta and lambda of the rows
  if (wave == 0) {
    const int t = t0 + lane;
    const float g = (p.decay == 1 && t < T) ? p.g[seq0 + (size_t)t * H] : 0.f;
    sGs[lane] = wave_incl_scan(g);
  } else if (wave == 1) {
    const int t = t0 + lane;
    const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
    sBeta[lane] = t < T ? p.beta[tok] : 0.f;
    sLam[lane] = p.qmix == 2 ? p.lam[tok] : (p.qmix ? p.lam[hh] : 0.f);
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int e = tid + NTHR * u, r = e / (DK / 8), c8 = (e % (DK / 8)) * 8;
    const bool ok = t0 + r < T;
    *reinterpret_cast<bf16x8*>(sKr + r * SR + c8) = ok ? rk[u] : bf16x8{};
    *reinterpret_cast<bf16x8*>(sQr + r * SR + c8) = ok ? rq[u] : bf16x8{};
  }
  __syncthreads();
  // ---- K K^T and Q K^T: tile pair pr = wave + 4 t (t < 3, pr < 10) of the
  // ten (I >= J) in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ..;
  // 32-wide k-steps, both operands 16-byte reads of rows
  const int g = lane >> 4, l16 = lane & 15;
  auto tile_I = [](int pr) { return pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3; };
  auto tile_J = [](int pr) { return pr - (pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 3 : 6); };
  f32x4 mK[3], mQ[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    mK[t] = mQ[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int pr = wave + 4 * t;
    if (pr >= 10) continue;  // wave-uniform
    const int I = tile_I(pr), J = tile_J(pr);
#pragma unroll
    for (int m = 0; m < DK / 32; ++m) {
      const int o = l16 * SR + 32 * m + 8 * g;
      const bf16x8 bk = *reinterpret_cast<const bf16x8*>(sKr + 16 * J * SR + o);
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(sKr + 16 * I * SR + o);
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQr + 16 * I * SR + o);
      mK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bk, mK[t], 0, 0, 0);
      mQ[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, mQ[t], 0, 0, 0);
    }
  }
  __syncthreads();  // the rows are no longer read (the inverse's arrays take their place)
  // ---- T to LDS (dense, zeros above the mask), Aqk to the record: lane
  // rows 16 I + 4 g + r, column 16 J + l16
  float* recA = ws.A + ch * CH * CH;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int pr = wave + 4 * t;
    if (pr >= 10) continue;
    const int I = tile_I(pr), J = tile_J(pr), j = 16 * J + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * g + r;
      const float d = fexp(fminf(sGs[i] - sGs[j], 0.f));
      const float e = sBeta[i] * __builtin_fmaf(sLam[i], mQ[t][r], mK[t][r]);
      sT[i * HP + j] = j < i ? e * d : 0.f;
      recA[i * CH + j] = j <= i ? mQ[t][r] * d : 0.f;
    }
  }
  // the six tiles above the diagonal are zero in the record (the inverse
  // reads none of them)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int u = wave + 4 * t;
    if (u >= 6) continue;
    const int I = u < 3 ? 0 : u < 5 ? 1 : 2, J = u < 3 ? u + 1 : u < 5 ? u - 1 : 3, j = 16 * J + l16;
#pragma unroll
    for (int r = 0; r < 4; ++r) recA[(16 * I + 4 * g + r) * CH + j] = 0.f;
  }
  __syncthreads();
  prep_inverse<HP>(sT, sAi, sP, ws.T + ch * CH * CH, tid);
}

// sum over the four lanes of each quad (DPP quad permutations), every lane
// gets the total
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));  // lane ^ 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, true));  // lane ^ 2
  return x;
}

// ---- pass 2 -----------------------------------------------------------------
template <int DK, int DVS>
struct PlainRecLay {
  static constexpr int SP = DVS + 4;  // row stride (floats) of [rows][DVS] arrays: 16-byte rows
  static constexpr int TP = CH + 1;   // row stride of the [64][64] arrays
  static constexpr int oS = 0;                // [DK][SP] state slice
  static constexpr int oA = oS + DK * SP;     // [64][TP] A (T under the per-value-channel beta)
  static constexpr int oAq = oA + CH * TP;    // [64][TP] Aqk
  static constexpr int oZ = oAq + CH * TP;    // [64][SP] written values z
  static constexpr int oM = oZ + CH * SP;     // [64][SP] erase multiplier M
  static constexpr int oW = oM + CH * SP;     // [64][SP] W
  static constexpr int oES = oW + CH * SP;    // [64][SP] E_bar S, or R = Z - E_bar S
  static constexpr int oQS = oES + CH * SP;   // [64][SP] Q_gamma S
  static constexpr int TOTAL = oQS + CH * SP;
  static_assert(2 * TOTAL * 4 <= 160 * 1024, "two workgroups per CU");
};

template <int DK, int DVS>
constexpr int plain_rec_lds_bytes() {
  return PlainRecLay<DK, DVS>::TOTAL * 4;
}

template <class IO, int DK, int DVS, bool REC = false>
__global__ __launch_bounds__(NTHR) void plain_rec_kernel(ChunkParams p, BwdWs ws) {
  using L = PlainRecLay<DK, DVS>;
  constexpr int SP = L::SP, TP = L::TP;
  static_assert(DVS == 16, "row ri x 4 columns per thread; 16 columns x 16 lanes in the substitution");
  __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
  float* sS = lds + L::oS;
  float* sA = lds + L::oA;
  float* sAq = lds + L::oAq;
  float* sZ = lds + L::oZ;
  float* sM = lds + L::oM;
  float* sW = lds + L::oW;
  float* sES = lds + L::oES;
  float* sQS = lds + L::oQS;

  const int tid = threadIdx.x;
  // workgroup -> (batch, head, slice); blockIdx values that share a residue
  // mod 8 run on one XCD, so the slices of a head read its records from one L2
  int wid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int NS = p.nslices;
  const int bh = wid / NS, slice = wid - bh * NS;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H, DV = p.DV;
  const int vbase = slice * DVS;
  const int N = (T + CH - 1) / CH;
  const int erase = p.erase, write = p.write;
  const bool subst = erase == 2;  // per-value-channel beta: per-column systems
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* vg = reinterpret_cast<const IO*>(p.v);
  IO* og = reinterpret_cast<IO*>(p.o);

  for (int e = tid; e < DK * DVS; e += NTHR) {
    const int c = e / DVS, v = e - c * DVS;
    sS[c * SP + v] = p.state_in ? p.state_in[((size_t)bh * DK + c) * DV + vbase + v] : 0.f;
  }

  // row layouts: thread = row ri x columns vq .. vq + 3 (quad member cq) for
  // the row products; the channel sums of E_bar S and Q_gamma S are split
  // over the quad (channels DK / 4 cq ..) and summed across it.  Update:
  // channel cu x VPT columns.
  const int ri = tid >> 2, cq = tid & 3, vq = 4 * cq;
  const int jend = ((tid >> 6) + 1) * 16;  // the wave's rows are 16 (tid / 64) .. + 15
  constexpr int CPQ = DK / 4;              // channels per quad member
  constexpr int TPC = NTHR / DK, VPT = DVS / TPC;
  const int cu = tid / TPC, vu = (tid % TPC) * VPT;

  for (int n = 0; n < N; ++n) {
    const int t0 = n * CH;
    const size_t ch = (size_t)bh * N + n;
    __syncthreads();  // the previous chunk's update of S and reads of W are complete
    if constexpr (REC) {
      for (int e = tid; e < DK * DVS; e += NTHR) {
        const int c = e / DVS, v = e - c * DVS;
        ws.S[(ch * DK + c) * DV + vbase + v] = sS[c * SP + v];
      }
    }
    // ---- every load of the phase first: A (or T), Aqk, this thread's
    // channels of its E_bar and Q_gamma rows, and z, M of its row and columns
    f32x4 ra[4], rq[4], e4[CPQ / 4], q4[CPQ / 4];
    float rv[4], rw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = *reinterpret_cast<const f32x4*>(ws.T + ch * CH * CH + 4 * (tid + NTHR * u));
      if constexpr (!REC) rq[u] = *reinterpret_cast<const f32x4*>(ws.A + ch * CH * CH + 4 * (tid + NTHR * u));
    }
    {
      const float* ebr = ws.Eb + (ch * CH + ri) * DK + CPQ * cq;
      const float* qgr = ws.Qg + (ch * CH + ri) * DK + CPQ * cq;
#pragma unroll
      for (int u = 0; u < CPQ / 4; ++u) {
        e4[u] = *reinterpret_cast<const f32x4*>(ebr + 4 * u);
        q4[u] = *reinterpret_cast<const f32x4*>(qgr + 4 * u);
      }
      const size_t tok = seq0 + (size_t)min(t0 + ri, T - 1) * H;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        rv[u] = ldf(vg + tok * DV + vbase + vq + u);
        rw[u] = subst ? p.beta[tok * DV + vbase + vq + u]
                      : (write == 1 ? p.w[tok * DV + vbase + vq + u] : p.beta[tok]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * (tid + NTHR * u), r = e / CH, c = e - r * CH;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sA[r * TP + c + i] = ra[u][i];
        if constexpr (!REC) sAq[r * TP + c + i] = rq[u][i];
      }
    }
    // ---- E_bar S and Q_gamma S of row ri: partial sums over the thread's
    // channels for all 16 columns, summed across the quad ---------------------
    {
      float es[DVS], qs[DVS];
#pragma unroll
      for (int v = 0; v < DVS; ++v) es[v] = qs[v] = 0.f;
#pragma unroll
      for (int u = 0; u < CPQ / 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* srow = sS + (CPQ * cq + 4 * u + i) * SP;
#pragma unroll
          for (int x = 0; x < DVS; x += 4) {
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(srow + x);
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              es[x + y] = __builtin_fmaf(e4[u][i], s4[y], es[x + y]);
              qs[x + y] = __builtin_fmaf(q4[u][i], s4[y], qs[x + y]);
            }
          }
        }
#pragma unroll
      for (int v = 0; v < DVS; ++v) {
        es[v] = quad_sum(es[v]);
        qs[v] = quad_sum(qs[v]);
      }
      // this thread's four columns (static selects over the quad member)
      f32x4 e_m, q_m;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        e_m[y] = cq == 0 ? es[y] : cq == 1 ? es[4 + y] : cq == 2 ? es[8 + y] : es[12 + y];
        q_m[y] = cq == 0 ? qs[y] : cq == 1 ? qs[4 + y] : cq == 2 ? qs[8 + y] : qs[12 + y];
      }
      const bool ok = t0 + ri < T;
      f32x4 z, m;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        z[y] = ok ? rw[y] * rv[y] : 0.f;
        m[y] = (ok && subst) ? rw[y] : 1.f;
      }
      *reinterpret_cast<f32x4*>(sQS + ri * SP + vq) = q_m;
      if (subst) {
        *reinterpret_cast<f32x4*>(sES + ri * SP + vq) = e_m;
        *reinterpret_cast<f32x4*>(sZ + ri * SP + vq) = z;
        *reinterpret_cast<f32x4*>(sM + ri * SP + vq) = m;
      } else {
        *reinterpret_cast<f32x4*>(sES + ri * SP + vq) = z - e_m;  // R = Z - E_bar S
      }
    }
    // K_tail column cu of the chunk for the update, requested here so that it
    // arrives during W and O
    float kt[CH];
    {
      const float* ktc = ws.Kt + ch * CH * DK + cu;
#pragma unroll
      for (int j = 0; j < CH; ++j) kt[j] = ktc[j * DK];
    }
    __syncthreads();
    // ---- W ---------------------------------------------------------------------
    if (!subst) {
      // W = A R: row ri, columns vq .. (A is zero above the diagonal, so the
      // wave runs to its last row)
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int j = 0; j < jend; ++j) w += sA[ri * TP + j] * *reinterpret_cast<const f32x4*>(sES + j * SP + vq);
      *reinterpret_cast<f32x4*>(sW + ri * SP + vq) = w;
      if constexpr (REC) *reinterpret_cast<f32x4*>(ws.W + (ch * CH + ri) * DV + vbase + vq) = w;
    } else {
      // forward substitution, column v = tid / 16, lanes split j
      const int v = tid >> 4, part = tid & 15;
      float wreg[4] = {0.f, 0.f, 0.f, 0.f};  // W[part + 16 m][v]
      for (int i = 0; i < CH; ++i) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int j = part + 16 * m;
          if (j < i) s = __builtin_fmaf(sA[i * TP + j], wreg[m], s);
        }
        s = sum16(s);
        const float w = sZ[i * SP + v] - sM[i * SP + v] * (sES[i * SP + v] + s);
        if ((i & 15) == part) wreg[i >> 4] = w;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sW[(part + 16 * m) * SP + v] = wreg[m];
        if constexpr (REC) ws.W[(ch * CH + part + 16 * m) * DV + vbase + v] = wreg[m];
      }
    }
    __syncthreads();
    // ---- O = Q_gamma S + Aqk W ---------------------------------------------------
    if constexpr (!REC) {
      f32x4 o = *reinterpret_cast<const f32x4*>(sQS + ri * SP + vq);
#pragma unroll 4
      for (int j = 0; j < jend; ++j) o += sAq[ri * TP + j] * *reinterpret_cast<const f32x4*>(sW + j * SP + vq);
      const int t = t0 + ri;
      if (t < T) {
        IO* op = og + (seq0 + (size_t)t * H) * DV + vbase + vq;
#pragma unroll
        for (int u = 0; u < 4; ++u) op[u] = (IO)o[u];
      }
    }
    // ---- S <- Diag(gamma_C) S + K_tail^T W: channel cu, columns vu .. -------
    {
      const float gC = ws.gC[ch * DK + cu];
      float s[VPT];
#pragma unroll
      for (int u = 0; u < VPT; ++u) s[u] = gC * sS[cu * SP + vu + u];
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int x = 0; x < VPT; x += 4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(sW + j * SP + vu + x);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[x + i] = __builtin_fmaf(kt[j], w4[i], s[x + i]);
        }
#pragma unroll
      for (int u = 0; u < VPT; ++u) sS[cu * SP + vu + u] = s[u];
    }
  }
  __syncthreads();
  if (p.state_out) {
    for (int e = tid; e < DK * DVS; e += NTHR) {
      const int c = e / DVS, v = e - c * DVS;
      p.state_out[((size_t)bh * DK + c) * DV + vbase + v] = sS[c * SP + v];
    }
  }
}

}  // namespace gdr

namespace gdr {

// ---- pass 2 on the matrix cores ---------------------------------------------
// The same recurrence on the matrix cores, for every gate kind but the
// per-value-channel beta: one workgroup of eight waves per (batch, head,
// 64-column slice).
// Waves 0-3 compute: wave w owns columns 16 w .. + 15 and the state S of
// those columns in accumulators: register r of block b of lane l holds
// S[16 b + 4 (l / 16) + r][16 w + l % 16].
//
// Every product runs in split precision (three bf16 MFMAs, at a sixth of the
// fp32 matrix instructions' time): the state, R, W and the other
// accumulator tiles serve as B operands once split, and the A operands are
// rows stored in kpos order, one 16-byte LDS read per half and fragment:
//   ES, QS  = E_bar S, Q_gamma S          A = E_bar, Q_gamma rows (token x channel)
//   W       = A (Z - ES)                  A = A rows (token x token), lower blocks only
//   O       = QS + Aqk W                  A = Aqk rows
//   S      <- Diag(gamma_C) S + K_tail^T W   A = K_tail^T rows (channel x token)
// Waves 4-7 stage a chunk's records in LDS in two sets, each written while
// the computing waves read the other: set B (K_tail^T, transposed on the way,
// and gamma_C) of chunk n while they form W and O of chunk n, set A (E_bar,
// Q_gamma, A, Aqk) of chunk n + 1 while they update the state; the staging
// waves also split each record value into its two halves.  Each set's
// inputs are loaded into the staging waves' registers a phase before they
// are staged.  A computing wave and a staging wave share each SIMD, so the
// staging arithmetic runs beside the MFMAs instead of between them.
template <int DK>
struct PlainMrecLay {
  // bf16 rows (elements), hi and lo arrays of each operand; 16-row fragment
  // reads of 16 bytes fall in distinct banks
  static constexpr int SE = DK + 8;  // E_bar, Q_gamma: [64][SE]
  static constexpr int SA = CH + 8;  // A, Aqk: [64][SA]; K_tail^T: [DK][SA]
  static constexpr int szE = CH * SE, szA = CH * SA, szK = DK * SA;  // elements per half
  static constexpr int oEb = 0, oQg = oEb + 2 * szE, oKtT = oQg + 2 * szE;  // bf16 offsets
  static constexpr int oA = oKtT + 2 * szK, oAq = oA + 2 * szA, oEnd = oAq + 2 * szA;
  static constexpr int oGC = oEnd * 2;  // bytes: gamma_C [DK] fp32
  static constexpr int BYTES = oGC + DK * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert((oGC % 16) == 0 && (SE * 2) % 16 == 0 && (SA * 2) % 16 == 0, "alignment");
};


template <int DK>
constexpr int plain_mrec_lds_bytes() {
  return PlainMrecLay<DK>::BYTES;
}

// Under a scalar decay (or none) the factor rows of a chunk are row scalings
// of the inputs, so the passes that read them form them while staging,
// instead of reading 96 KB per chunk (dk = 128) back from the workspace:
//   E_bar_t = gamma_t e_t,  Q_gamma_t = gamma_t q_t,  K_tail_t = (gamma_C / gamma_t) k_t,
//   e_t = beta_t (k_t + lam_t q_t), or b_t (.) k_t,  gamma_t = exp(G_t),
// G the chunk's prefix sum of the log-decay (zero past T), with the prep's
// operations (so these are the rows it would have written).  SdLane: the
// log-decay, beta and lambda of token t0 + lane of the chunk.
struct SdLane {
  float g, beta, lam;
};
// (every load is unconditional, a scalar the gate kinds do not use read from
// k, which is always there and holds at least four bytes per token: a value
// chosen by a branch would make the wave wait for its load at the branch's
// join; the flags select at use, in sd_scan and sd_rows)
__device__ __forceinline__ SdLane sd_lane_load(const ChunkParams& p, size_t seq0, int t0, int hh, int lane) {
  const size_t tok = seq0 + (size_t)min(t0 + lane, p.T - 1) * p.H;
  const float* any = reinterpret_cast<const float*>(p.k);
  const float* gp = p.decay == 1 ? p.g : any;
  const float* bp = p.erase == 0 ? p.beta : any;
  const float* lp = p.qmix == 2 ? p.lam + tok : (p.qmix ? p.lam + hh : any + tok);
  return SdLane{gp[tok], bp[tok], *lp};
}
// G_{t0 + lane} in lane lane (every lane of the wave active)
__device__ __forceinline__ float sd_scan(const ChunkParams& p, const SdLane& s, int t0, int lane) {
  return wave_incl_scan((p.decay == 1 && t0 + lane < p.T) ? s.g : 0.f);
}
// E_bar and Q_gamma of four channels of chunk token t from the raw k, q (and
// b) of those channels (every lane active: the token's scalars come by
// lane shuffles)
__device__ __forceinline__ void sd_rows(const ChunkParams& p, float G, const SdLane& s, int t, int t0, f32x4 k,
                                        f32x4 q, f32x4 b, f32x4& eb, f32x4& qg) {
  const float Gt = __shfl(G, t), bt = __shfl(s.beta, t), lt = p.qmix ? __shfl(s.lam, t) : 0.f;
  const bool ok = t0 + t < p.T;
  const float gam = fexp(Gt);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float kv = ok ? k[i] : 0.f, qv = ok ? q[i] : 0.f;
    float ev = p.erase == 1 ? b[i] * kv : bt * __builtin_fmaf(lt, qv, kv);
    if (!ok) ev = 0.f;
    eb[i] = ev * gam;
    qg[i] = qv * gam;
  }
}
// K_tail of four channels of chunk token t
__device__ __forceinline__ f32x4 sd_ktail(const ChunkParams& p, float G, float GC, int t, int t0, f32x4 k) {
  const float Gt = __shfl(G, t);
  const bool ok = t0 + t < p.T;
  f32x4 kt;
#pragma unroll
  for (int i = 0; i < 4; ++i) kt[i] = (ok ? k[i] : 0.f) * fexp(GC - Gt);
  return kt;
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// SD: a scalar decay or none; the factor rows are formed from the inputs
// (sd_rows) rather than read from the workspace.
template <class IO, int DK, bool REC = false, bool SD = false>
__global__ __launch_bounds__(2 * NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void plain_mrec_kernel(ChunkParams p, BwdWs ws) {
  using L = PlainMrecLay<DK>;
  constexpr int SE = L::SE, SA = L::SA, NB = DK / 16;
  constexpr int DVS = 64;
  constexpr int NQ_E = CH * DK / 4 / NTHR;  // 16-byte pieces per staging thread of a [64][DK] record array
  constexpr int NQ_A = CH * CH / 4 / NTHR;  // of a [64][64] array
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  bf16* sEb = reinterpret_cast<bf16*>(lds) + L::oEb;  // hi, then lo at + szE
  bf16* sQg = reinterpret_cast<bf16*>(lds) + L::oQg;
  bf16* sKtT = reinterpret_cast<bf16*>(lds) + L::oKtT;  // hi, then lo at + szK
  bf16* sA = reinterpret_cast<bf16*>(lds) + L::oA;      // hi, then lo at + szA
  bf16* sAq = reinterpret_cast<bf16*>(lds) + L::oAq;
  float* sGC = reinterpret_cast<float*>(lds + L::oGC);
  constexpr int hE = L::szE, hA = L::szA, hK = L::szK;

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
  const int N = (T + CH - 1) / CH;
  const size_t seq0 = (size_t)bb * T * H + hh;

  if (wave >= 4) {
    // ================= staging waves =================
    const int st = tid - NTHR, sw = wave - 4;  // thread and wave within the staging group
    const int qj = lane & 3, qk = lane >> 2;
    const IO* kin = reinterpret_cast<const IO*>(p.k);
    const IO* qin = reinterpret_cast<const IO*>(p.q);
    // set A: E_bar, Q_gamma (SD: from the raw k, q and the per-channel erase
    // gate), A, Aqk (the record mode reads neither Q_gamma nor Aqk); set B:
    // K_tail (SD: from the raw k), gamma_C.  The pieces
    // of the [64][DK] arrays are in the quad layout: lane (k, j) = (lane / 4,
    // lane % 4) of staging wave w takes token 4 t4 + j, channels 4 k .. + 3 of
    // a block of 4 tokens x 64 channels, E_bar and Q_gamma as row pieces and
    // K_tail through the quad transpose (channel 4 k + j, tokens 4 t4 .. + 3
    // as one 16-byte LDS write; the wave's 64 channel rows fall in distinct
    // banks).
    struct RecA {
      typename Raw<IO>::v4 kr[SD ? NQ_E : 1], qr[SD ? NQ_E : 1];
      f32x4 eb[SD ? 1 : NQ_E], qg[SD ? 1 : NQ_E], bq[SD ? NQ_E : 1], a[NQ_A], aq[REC ? 1 : NQ_A];
      SdLane sd;
    };
    struct RecB {
      typename Raw<IO>::v4 kr[SD ? NQ_E : 1];
      f32x4 kt[SD ? 1 : NQ_E];
      float gc;
      SdLane sd;
    };
    auto piece = [&](int u, int& t, int& c) __attribute__((always_inline)) {
      const int blk = sw + 4 * u;
      t = 4 * (blk / (DK / 64)) + qj;
      c = 64 * (blk % (DK / 64)) + 4 * qk;
    };
    auto load_a = [&](int n, RecA& R) __attribute__((always_inline)) {
      const size_t ch = (size_t)bh * N + n;
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        if constexpr (SD) {
          int t, c;
          piece(u, t, c);
          const size_t tokq = seq0 + (size_t)min(n * CH + t, T - 1) * H;
          R.kr[u] = ldraw4(kin + tokq * DK + c);
          R.qr[u] = ldraw4(qin + tokq * DK + c);
          if (p.erase == 1) R.bq[u] = *reinterpret_cast<const f32x4*>(p.b + tokq * DK + c);
        } else {
          const size_t o = ch * CH * DK + 4 * (st + NTHR * u);
          R.eb[u] = *reinterpret_cast<const f32x4*>(ws.Eb + o);
          if constexpr (!REC) R.qg[u] = *reinterpret_cast<const f32x4*>(ws.Qg + o);
        }
      }
      if constexpr (SD) R.sd = sd_lane_load(p, seq0, n * CH, hh, lane);
#pragma unroll
      for (int u = 0; u < NQ_A; ++u) {
        const size_t o = ch * CH * CH + 4 * (st + NTHR * u);
        R.a[u] = *reinterpret_cast<const f32x4*>(ws.T + o);
        if constexpr (!REC) R.aq[u] = *reinterpret_cast<const f32x4*>(ws.A + o);
      }
    };
    auto load_b = [&](int n, RecB& R) __attribute__((always_inline)) {
      const size_t ch = (size_t)bh * N + n;
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        int t, c;
        piece(u, t, c);
        if constexpr (SD) R.kr[u] = ldraw4(kin + (seq0 + (size_t)min(n * CH + t, T - 1) * H) * DK + c);
        else R.kt[u] = *reinterpret_cast<const f32x4*>(ws.Kt + ch * CH * DK + (size_t)t * DK + c);
      }
      if constexpr (SD) R.sd = sd_lane_load(p, seq0, n * CH, hh, lane);
      else R.gc = st < DK ? ws.gC[ch * DK + st] : 0.f;
    };
    auto stage_a = [&](const RecA& R, int t0) __attribute__((always_inline)) {
      float G = 0.f;
      if constexpr (SD) G = sd_scan(p, R.sd, t0, lane);
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        if constexpr (SD) {
          int tq, cq4;
          piece(u, tq, cq4);
          f32x4 eb, qgm;
          sd_rows(p, G, R.sd, tq, t0, widen(R.kr[u]), widen(R.qr[u]), R.bq[u], eb, qgm);
          put_split<SE>(sEb, hE, tq, cq4, eb);
          if constexpr (!REC) put_split<SE>(sQg, hE, tq, cq4, qgm);
        } else {
          const int e = 4 * (st + NTHR * u), t = e / DK, c = e - t * DK;
          put_split<SE>(sEb, hE, t, c, R.eb[u]);
          if constexpr (!REC) put_split<SE>(sQg, hE, t, c, R.qg[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < NQ_A; ++u) {
        const int e = 4 * (st + NTHR * u), t = e / CH, c = e - t * CH;
        put_split<SA>(sA, hA, t, c, R.a[u]);
        if constexpr (!REC) put_split<SA>(sAq, hA, t, c, R.aq[u]);
      }
    };
    auto stage_b = [&](const RecB& R, int t0) __attribute__((always_inline)) {
      float G = 0.f, GC = 0.f;
      if constexpr (SD) {
        G = sd_scan(p, R.sd, t0, lane);
        GC = lane_value(G, 63);
      }
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        const int blk = sw + 4 * u, t4 = blk / (DK / 64), cq = 64 * (blk % (DK / 64)) + lane;
        f32x4 kt;
        if constexpr (SD) {
          int tq, cq4;
          piece(u, tq, cq4);
          kt = sd_ktail(p, G, GC, tq, t0, widen(R.kr[u]));
        } else {
          kt = R.kt[u];
        }
        put_split<SA>(sKtT, hK, cq, 4 * t4, quad_transpose(kt, qj));
      }
      if (st < DK) sGC[st] = SD ? fexp(GC) : R.gc;
    };

    RecA Ra;
    RecB Rb;
    if (N > 0) {
      load_a(0, Ra);
      load_b(0, Rb);
      stage_a(Ra, 0);
    }
    __syncthreads();  // set A of the first chunk is staged
    for (int n = 0; n < N; ++n) {
      // phase 1 of chunk n (the computing waves read set A): set B of chunk n
      if (n + 1 < N) load_a(n + 1, Ra);
      stage_b(Rb, n * CH);
      __syncthreads();
      // phase 2 of chunk n (they read set B): set A of chunk n + 1
      if (n + 1 < N) {
        load_b(n + 1, Rb);
        stage_a(Ra, (n + 1) * CH);
      }
      __syncthreads();
    }
    return;
  }

  // ================= computing waves =================
  const int write = p.write;
  const int col = slice * DVS + 16 * wave + l16;  // this lane's value column
  const IO* vg = reinterpret_cast<const IO*>(p.v);
  IO* og = reinterpret_cast<IO*>(p.o);
  f32x4 S[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[b][r] = p.state_in ? p.state_in[((size_t)bh * DK + 16 * b + 4 * g + r) * DV + col] : 0.f;
  // this lane's z inputs, rows 16 I + 4 g + r of its column, a chunk ahead
  IO v[16];
  float gt[16];
  auto load_z = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const size_t tok = seq0 + (size_t)min(n * CH + 16 * (k >> 2) + 4 * g + (k & 3), T - 1) * H;
      v[k] = vg[tok * DV + col];
      gt[k] = *(write == 1 ? p.w + tok * DV + col : p.beta + tok);  // (one load either way)
    }
  };
  if (N > 0) load_z(0);
  __syncthreads();  // set A of the first chunk is staged
  for (int n = 0; n < N; ++n) {
    const int t0 = n * CH;
    const size_t ch = (size_t)bh * N + n;
    float z[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool ok = t0 + 16 * (k >> 2) + 4 * g + (k & 3) < T;  // row 16 I + 4 g + r, k = 4 I + r
      z[k] = ok ? gt[k] * (float)v[k] : 0.f;
    }
    if (n + 1 < N) load_z(n + 1);
    // ---- ES, QS -----------------------------------------------------------------
    constexpr int NKS = DK / 32;
    SplitB Sb[NKS];
#pragma unroll
    for (int m = 0; m < NKS; ++m) Sb[m] = split_b(S[2 * m], S[2 * m + 1]);
    f32x4 R[4], QS[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 es = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NKS; ++m) {
        es = mma_split(sEb + (16 * I + l16) * SE + 32 * m + 8 * g, hE, Sb[m], es);
        if constexpr (!REC) qs = mma_split(sQg + (16 * I + l16) * SE + 32 * m + 8 * g, hE, Sb[m], qs);
      }
      QS[I] = qs;
      // R = Z - E_bar S (rows 16 I + 4 g + r of this lane's column)
#pragma unroll
      for (int r = 0; r < 4; ++r) R[I][r] = z[4 * I + r] - es[r];
    }
    // ---- W = A R (row block I takes the k-steps of tokens below 32 (I / 2 + 1)) ---
    SplitB Rb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) Rb[q] = split_b(R[2 * q], R[2 * q + 1]);
    f32x4 W[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q <= I / 2; ++q) w = mma_split(sA + (16 * I + l16) * SA + 32 * q + 8 * g, hA, Rb[q], w);
      W[I] = w;
    }
    SplitB Wb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) Wb[q] = split_b(W[2 * q], W[2 * q + 1]);
    if constexpr (REC) {
      // W and the entering state S to the workspace, issued after the chain's
      // products (stored at the top of the step they delayed them)
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) ws.W[(ch * CH + 16 * I + 4 * g + r) * DV + col] = W[I][r];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) ws.S[(ch * DK + 16 * b + 4 * g + r) * DV + col] = S[b][r];
    } else {
      // ---- O = QS + Aqk W -------------------------------------------------------
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 o = QS[I];
#pragma unroll
        for (int q = 0; q <= I / 2; ++q) o = mma_split(sAq + (16 * I + l16) * SA + 32 * q + 8 * g, hA, Wb[q], o);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + 16 * I + 4 * g + r;
          if (t < T) og[(seq0 + (size_t)t * H) * DV + col] = (IO)o[r];
        }
      }
    }
    __syncthreads();  // set B of this chunk is staged; set A is free
    // ---- S <- Diag(gamma_C) S + K_tail^T W ---------------------------------------
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4 gc = *reinterpret_cast<const f32x4*>(sGC + 16 * b + 4 * g);
      f32x4 s = S[b] * gc;
#pragma unroll
      for (int q = 0; q < 2; ++q) s = mma_split(sKtT + (16 * b + l16) * SA + 32 * q + 8 * g, hK, Wb[q], s);
      S[b] = s;
    }
    __syncthreads();  // set A of the next chunk is staged; set B is free
  }
  if (p.state_out) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.state_out[((size_t)bh * DK + 16 * b + 4 * g + r) * DV + col] = S[b][r];
  }
}

}  // namespace gdr
