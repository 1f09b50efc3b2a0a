// Backward of the chunkwise forward: gradients of every input for given
// cotangents dO of the outputs and dS of the final state.
//
// The chunk form's backward of "Gated DeltaNet-2: Decoupling Erase and
// Write in Linear Attention" (key design 3): per chunk, the gradient of the
// triangular inverse is dT = -tril(A^T dA A^T, -1), and with the per-channel
// gates the gate weights stay inside the dA products (no scalar can be
// pulled out of them).  Evaluated here on the regrouped forward of the plain
// kernel (W = A R, R = Z - E_bar S), where dA = dW R^T and therefore
//   dR = A^T dW,   dT = -tril(dR W^T, -1),   dZ = dR,   dE_bar = -dR S^T.
// Accumulation is fp32; the products of the record recurrence, the state
// pass and the product pass run in split precision (each fp32 operand as
// bf16 hi and lo halves, Xhi Yhi + Xhi Ylo + Xlo Yhi on the bf16 matrix
// cores), the key pass on fp32 MFMAs.  Four passes, each a kernel on the
// caller's stream:
//
//  0  record  the two-pass plain forward in record mode
//             (plain_split_kernel.hpp): per chunk A = (I + T)^{-1} (in the
//             place of T), A_qk, E_bar, Q_gamma, K_tail, gamma_C, and per slice
//             the entering state S and W, to the workspace.
//  A  state   per (batch, head, 64-column slice), chunks in reverse, the
//             gradient of the state dS (leaving the chunk) carried in MFMA
//             accumulators:
//               dW = A_qk^T dO + K_tail dS
//               dR = A^T dW,  A = (I + T)^{-1} from the record pass
//               dS <- Diag(gamma_C) dS + Q_gamma^T dO - E_bar^T dR
//             writes dR and each chunk's incoming dS; the last dS is the
//             gradient of the initial state.
//  B1 prod    per (batch, head, chunk): the products over the value channels
//               dT = -tril(dR W^T, -1), dA_qk = tril(dO W^T),
//               dE_bar = -dR S^T, dQ_gamma = dO S^T, dK_tail = W dS^T,
//               sC = rowsum(S (.) dS)
//  B2 key     per (batch, head, chunk): the decay-weighted sums back to the
//             rows, with d_ij[c] = exp(G_i[c] - G_j[c]) <= 1,
//               de_i  = gamma_i dE_bar_i + sum_{j<i}  dT[i][j]  k_j d_ij
//               dq_i  = gamma_i dQ_gamma_i + sum_{j<=i} dA_qk[i][j] k_j d_ij
//               dk_j  = tail_j dK_tail_j + sum_{i>j} dT[i][j] e_i d_ij + sum_{i>=j} dA_qk[i][j] q_i d_ij
//               dG_i  = e_i gamma_i dE_bar_i + q_i gamma_i dQ_gamma_i + e_i P_i + q_i Pq_i - k_i (R_i + Rq_i)
//             then dg_t = sum_{r>=t} dG_r + sum_{j<t} K_tail_j dK_tail_j + gamma_C sC:
//             K_tail_j depends on g_t for j < t <= 63 and gamma_C on every
//             g_t of the chunk, so these enter as a prefix sum and a constant
//             instead of as pairs of O(1) terms at rows j and 63 that cancel
//             (in a ragged tail the last valid row has tail = 1); the
//             diagonal of A_qk (d_ii = 1) likewise stays out of dG.  Then the
//             gate chain (e = beta (k + lambda q) or b (.) k; z = beta v or w (.) v).
// A lambda shared by a head's tokens sums its per-token gradients in a
// final reduction.
#pragma once

#include "plain_kernel.hpp"
#include "plain_split_kernel.hpp"

namespace gdr {



// rows x COLS fp32 from global memory (row stride COLS) to LDS (row stride
// LD), four floats per load, the loads of up to 8 quads per thread issued
// together
template <int ROWS, int COLS, int LD>
__device__ __forceinline__ void copy_rows(float* dst, const float* src, int tid) {
  constexpr int QPR = COLS / 4, NQ = ROWS * QPR / NTHR, UB = NQ < 8 ? NQ : 8;
  static_assert(NQ * NTHR == ROWS * QPR && NQ % UB == 0, "copy layout");
  for (int u0 = 0; u0 < NQ; u0 += UB) {
    f32x4 x[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) x[u] = *reinterpret_cast<const f32x4*>(src + (size_t)(tid + NTHR * (u0 + u)) * 4);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int e = tid + NTHR * (u0 + u), r = e / QPR, c4 = (e - r * QPR) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[r * LD + c4 + i] = x[u][i];
    }
  }
}

// ---- pass A: the reverse state recurrence, on the matrix cores ----------------
// One workgroup of eight waves per (batch, head, 64-column slice).  Waves 0-3
// compute on the matrix cores in split precision (bf16 hi and lo halves of
// each fp32 operand, three bf16 MFMAs per product, fp32 accumulation): wave w
// owns columns 16 w .. + 15 and dS of those columns in accumulators (register
// r of block b of lane l: dS[16 b + 4 (l / 16) + r][16 w + l % 16], the
// forward recurrence's state layout).  dS, dO, dW and dR serve as B operands
// once split, and the A operands are staged rows with their k index in the
// fragments' order (kpos), 16-byte LDS reads per half:
//   dW = A_qk^T dO + K_tail dS        A = A_qk^T rows, K_tail rows
//   dR = A^T dW                       A = A^T rows (upper blocks only)
//   dS <- Diag(gamma_C) dS + Q_gamma^T dO - E_bar^T dR   A = Q_gamma^T, E_bar^T rows
// Waves 4-7 stage a chunk's records in LDS (the transposes on the way; under
// a scalar decay the factor rows formed from the inputs) in two sets, each
// written while the computing waves read the other: set B (Q_gamma^T,
// E_bar^T, gamma_C) of chunk n during dW and dR of chunk n, set A (K_tail,
// A_qk^T, A^T) of chunk n - 1 during the state update of chunk n.  Each set's
// inputs are loaded into the staging waves' registers a phase before they
// are staged.  A computing wave and a staging wave share each SIMD, so the
// staging arithmetic runs beside the MFMAs instead of between them.
template <int DK>
struct BwdAMLay {
  // bf16 rows (elements); hi then lo array of each operand
  static constexpr int SE = DK + 8, SA = CH + 8;
  static constexpr int hKt = CH * SE, hA = CH * SA, hT = DK * SA;  // elements per half
  static constexpr int oKt = 0;                  // [64][SE] K_tail rows        (set A)
  static constexpr int oAqT = oKt + 2 * hKt;     // [64][SA] A_qk^T             (set A)
  static constexpr int oAT = oAqT + 2 * hA;      // [64][SA] A^T                (set A)
  static constexpr int oQgT = oAT + 2 * hA;      // [DK][SA] Q_gamma^T          (set B)
  static constexpr int oEbT = oQgT + 2 * hT;     // [DK][SA] E_bar^T            (set B)
  static constexpr int oGC = (oEbT + 2 * hT) * 2;  // bytes: [DK] gamma_C fp32   (set B)
  static constexpr int BYTES = oGC + DK * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(oGC % 16 == 0, "alignment");
};

// SD: a scalar decay or none; E_bar, Q_gamma, K_tail and gamma_C are formed
// from the inputs while staging (sd_rows) rather than read from the workspace.
template <class IO, int DK, bool SD = false>
__global__ __launch_bounds__(2 * NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_state_mfma_kernel(BwdParams p) {
  using L = BwdAMLay<DK>;
  constexpr int SE = L::SE, SA = L::SA, NB = DK / 16, DVS = 64;
  constexpr int NQ_E = CH * DK / 4 / NTHR, NQ_A = CH * CH / 4 / NTHR;
  constexpr int hKt = L::hKt, hA = L::hA, hT = L::hT;
  __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
  bf16* lb = reinterpret_cast<bf16*>(lds);
  bf16 *sKt = lb + L::oKt, *sQgT = lb + L::oQgT, *sEbT = lb + L::oEbT;
  bf16 *sAqT = lb + L::oAqT, *sAT = lb + L::oAT;
  float* sGC = reinterpret_cast<float*>(lds + L::oGC);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  int wid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int NS = p.f.DV / DVS;
  const int bh = wid / NS, slice = wid - bh * NS;
  const int bb = bh / p.f.H, hh = bh - bb * p.f.H;
  const int T = p.f.T, H = p.f.H, DV = p.f.DV, N = p.nchunks;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const BwdWs& ws = p.ws;

  if (wave >= 4) {
    // ================= staging waves =================
    const int st = tid - NTHR, sw = wave - 4;  // thread and wave within the staging group
    const int qj = lane & 3, qk = lane >> 2;
    const IO* kin = reinterpret_cast<const IO*>(p.f.k);
    const IO* qin = reinterpret_cast<const IO*>(p.f.q);
    // set A's inputs: K_tail (SD: the raw k), A, A_qk; set B's: E_bar and
    // Q_gamma (SD: the raw k, q and the per-channel erase gate), gamma_C.
    // E_bar, Q_gamma, A, A_qk are staged transposed: lane (k, j) = (lane / 4,
    // lane % 4) of staging wave w loads token 4 t4 + j, channels 4 k .. + 3
    // of a block of 4 tokens x 64 channels (rows stay 256-byte runs), the
    // quad transposes it, and the lane writes channel 4 k + j, tokens 4 t4 ..
    // + 3 as one 16-byte LDS write (64 consecutive channel rows per wave: no
    // bank conflicts).  K_tail stays row-major.
    struct RecA {
      typename Raw<IO>::v4 kr[SD ? NQ_E : 1];
      f32x4 kt[SD ? 1 : NQ_E], a[NQ_A], aq[NQ_A];
      SdLane sd;
    };
    struct RecB {
      typename Raw<IO>::v4 kr[SD ? NQ_E : 1], qr[SD ? NQ_E : 1];
      f32x4 eb[SD ? 1 : NQ_E], qg[SD ? 1 : NQ_E], bq[SD ? NQ_E : 1];
      float gc;
      SdLane sd;
    };
    // token and first channel of piece u of a [64][DK] array in the quad layout
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
          R.kr[u] = ldraw4(kin + (seq0 + (size_t)min(n * CH + t, T - 1) * H) * DK + c);
        } else {
          R.kt[u] = *reinterpret_cast<const f32x4*>(ws.Kt + ch * CH * DK + 4 * (st + NTHR * u));
        }
      }
      if constexpr (SD) R.sd = sd_lane_load(p.f, seq0, n * CH, hh, lane);
#pragma unroll
      for (int u = 0; u < NQ_A; ++u) {
        const int t = 4 * (sw + 4 * u) + qj, c = 4 * qk;
        const size_t o = ch * CH * CH + (size_t)t * CH + c;
        R.a[u] = *reinterpret_cast<const f32x4*>(ws.T + o);
        R.aq[u] = *reinterpret_cast<const f32x4*>(ws.A + o);
      }
    };
    auto load_b = [&](int n, RecB& R) __attribute__((always_inline)) {
      const size_t ch = (size_t)bh * N + n;
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        int t, c;
        piece(u, t, c);
        if constexpr (SD) {
          const size_t tokq = seq0 + (size_t)min(n * CH + t, T - 1) * H;
          R.kr[u] = ldraw4(kin + tokq * DK + c);
          R.qr[u] = ldraw4(qin + tokq * DK + c);
          if (p.f.erase == 1) R.bq[u] = *reinterpret_cast<const f32x4*>(p.f.b + tokq * DK + c);
        } else {
          const size_t o = ch * CH * DK + (size_t)t * DK + c;
          R.eb[u] = *reinterpret_cast<const f32x4*>(ws.Eb + o);
          R.qg[u] = *reinterpret_cast<const f32x4*>(ws.Qg + o);
        }
      }
      if constexpr (SD) R.sd = sd_lane_load(p.f, seq0, n * CH, hh, lane);
      else R.gc = st < DK ? ws.gC[ch * DK + st] : 0.f;
    };
    auto stage_a = [&](const RecA& R, int t0) __attribute__((always_inline)) {
      float G = 0.f, GC = 0.f;
      if constexpr (SD) {
        G = sd_scan(p.f, R.sd, t0, lane);
        GC = lane_value(G, 63);
      }
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        if constexpr (SD) {
          int tq, cq4;
          piece(u, tq, cq4);
          put_split<SE>(sKt, hKt, tq, cq4, sd_ktail(p.f, G, GC, tq, t0, widen(R.kr[u])));
        } else {
          const int e = 4 * (st + NTHR * u), t = e / DK, c = e - t * DK;
          put_split<SE>(sKt, hKt, t, c, R.kt[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < NQ_A; ++u) {
        const int t4 = sw + 4 * u, cq = 4 * qk + qj;
        put_split<SA>(sAT, hA, cq, 4 * t4, quad_transpose(R.a[u], qj));
        put_split<SA>(sAqT, hA, cq, 4 * t4, quad_transpose(R.aq[u], qj));
      }
    };
    auto stage_b = [&](const RecB& R, int t0) __attribute__((always_inline)) {
      float G = 0.f, GC = 0.f;
      if constexpr (SD) {
        G = sd_scan(p.f, R.sd, t0, lane);
        GC = lane_value(G, 63);
      }
#pragma unroll
      for (int u = 0; u < NQ_E; ++u) {
        const int blk = sw + 4 * u, t4 = blk / (DK / 64), cq = 64 * (blk % (DK / 64)) + 4 * qk + qj;
        f32x4 eb, qgm;
        if constexpr (SD) {
          int tq, cq4;
          piece(u, tq, cq4);
          sd_rows(p.f, G, R.sd, tq, t0, widen(R.kr[u]), widen(R.qr[u]), R.bq[u], eb, qgm);
        } else {
          eb = R.eb[u];
          qgm = R.qg[u];
        }
        put_split<SA>(sQgT, hT, cq, 4 * t4, quad_transpose(qgm, qj));
        put_split<SA>(sEbT, hT, cq, 4 * t4, quad_transpose(eb, qj));
      }
      if (st < DK) sGC[st] = SD ? fexp(GC) : R.gc;
    };

    RecA Ra;
    RecB Rb;
    if (N > 0) {
      load_b(N - 1, Rb);
      load_a(N - 1, Ra);
      stage_a(Ra, (N - 1) * CH);
    }
    __syncthreads();  // set A of the last chunk is staged
    for (int n = N - 1; n >= 0; --n) {
      // phase 1 of chunk n (the computing waves read set A): set B of chunk n
      if (n > 0) load_a(n - 1, Ra);
      stage_b(Rb, n * CH);
      __syncthreads();
      // phase 2 of chunk n (they read set B): set A of chunk n - 1
      if (n > 0) {
        load_b(n - 1, Rb);
        stage_a(Ra, (n - 1) * CH);
      }
      __syncthreads();
    }
    return;
  }

  // ================= computing waves =================
  const int col = slice * DVS + 16 * wave + l16;
  const IO* dog = reinterpret_cast<const IO*>(p.d_o);
  f32x4 dS[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dS[b][r] = p.d_st ? p.d_st[((size_t)bh * DK + 16 * b + 4 * g + r) * DV + col] : 0.f;
  // dO rows 16 I + 4 g + r of this lane's column, a chunk ahead
  IO o[16];
  auto load_o = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = n * CH + 16 * (k >> 2) + 4 * g + (k & 3);
      o[k] = dog[(seq0 + (size_t)min(t, T - 1) * H) * DV + col];
    }
  };
  if (N > 0) load_o(N - 1);
  __syncthreads();  // set A of the last chunk is staged
  for (int n = N - 1; n >= 0; --n) {
    const size_t ch = (size_t)bh * N + n;
    float dO[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) dO[k] = n * CH + 16 * (k >> 2) + 4 * g + (k & 3) < T ? (float)o[k] : 0.f;
    if (n > 0) load_o(n - 1);
    // the gradient of the state leaving this chunk, for the product pass
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) ws.dS[(ch * DK + 16 * b + 4 * g + r) * DV + col] = dS[b][r];
    // ---- dW = A_qk^T dO + K_tail dS (A_qk^T is zero below the diagonal) ---------
    // dO tiles (rows 16 J + 4 g + r) and dS as split B operands; row block I
    // of an upper-triangular factor takes the k-steps of tokens from 32 (I / 2)
    constexpr int NKS = DK / 32;
    SplitB dOb[2], dSb[NKS];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      dOb[q] = split_b(f32x4{dO[8 * q], dO[8 * q + 1], dO[8 * q + 2], dO[8 * q + 3]},
                       f32x4{dO[8 * q + 4], dO[8 * q + 5], dO[8 * q + 6], dO[8 * q + 7]});
#pragma unroll
    for (int m = 0; m < NKS; ++m) dSb[m] = split_b(dS[2 * m], dS[2 * m + 1]);
    f32x4 dW[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      // (the two products in two accumulators)
      f32x4 w = {0.f, 0.f, 0.f, 0.f}, w2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = I / 2; q < 2; ++q) w2 = mma_split(sAqT + (16 * I + l16) * SA + 32 * q + 8 * g, hA, dOb[q], w2);
#pragma unroll
      for (int m = 0; m < NKS; ++m) w = mma_split(sKt + (16 * I + l16) * SE + 32 * m + 8 * g, hKt, dSb[m], w);
      dW[I] = w + w2;
    }
    // ---- dR = A^T dW (A^T is zero below the diagonal) ------------------------------
    SplitB dWb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) dWb[q] = split_b(dW[2 * q], dW[2 * q + 1]);
    f32x4 dR[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 r4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = I / 2; q < 2; ++q) r4 = mma_split(sAT + (16 * I + l16) * SA + 32 * q + 8 * g, hA, dWb[q], r4);
      dR[I] = r4;
#pragma unroll
      for (int r = 0; r < 4; ++r) ws.dR[(ch * CH + 16 * I + 4 * g + r) * DV + col] = r4[r];
    }
    __syncthreads();  // set B of this chunk is staged; set A is free
    // ---- dS <- Diag(gamma_C) dS + Q_gamma^T dO - E_bar^T dR -----------------------
    // (dR negated once; the two products in two accumulators)
    SplitB ndRb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) ndRb[q] = split_b(-dR[2 * q], -dR[2 * q + 1]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const f32x4 gc = *reinterpret_cast<const f32x4*>(sGC + 16 * b + 4 * g);
      f32x4 sq = dS[b] * gc, se = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        sq = mma_split(sQgT + (16 * b + l16) * SA + 32 * q + 8 * g, hT, dOb[q], sq);
        se = mma_split(sEbT + (16 * b + l16) * SA + 32 * q + 8 * g, hT, ndRb[q], se);
      }
      dS[b] = sq + se;
    }
    __syncthreads();  // set A of the next chunk is staged; set B is free
  }
  if (p.dstate) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dstate[((size_t)bh * DK + 16 * b + 4 * g + r) * DV + col] = dS[b][r];
  }
}

// ---- pass B1: products over the value channels, on the matrix cores --------
// One workgroup of four waves per (batch, head, chunk), two per CU.  The value
// channels are taken in quarters of 32: dR, dO, W [64][32] and S, dS [DK][32]
// of the quarter in LDS (70 KB at DK = 128), the products' partial sums
// carried over the quarters in accumulators; while one workgroup waits for
// its loads, the other computes.  Wave w owns row block w (rows 16 w .. + 15)
// of every output: dT and dA_qk (blocks J <= w), dE_bar, dQ_gamma, dK_tail
// (all DK / 16 column blocks).  Every product contracts over the value
// channels in the split precision of plain_mrec_kernel: each fp32 operand is
// staged as bf16 hi and lo halves (row stride 40, the k index of every row in
// the fragments' order, kpos), and a quarter is one k-step of
// v_mfma_f32_16x16x32_bf16, three MFMAs per product (Xhi Yhi + Xhi Ylo +
// Xlo Yhi) with fp32 accumulation; both operands are 16-byte LDS reads of
// rows.  sC = sum_v S (.) dS per key channel is summed in fp32 from the
// staging registers.
template <int DK>
struct BwdB1Lay {
  static constexpr int VH = 32, SE = VH + 8;
  // rows of the staged operands, then the elements of one half
  static constexpr int rR = 0, rO = CH, rW = 2 * CH, rS = 3 * CH, rdS = 3 * CH + DK, NROW = 3 * CH + 2 * DK;
  static constexpr int HALF = NROW * SE;
  static constexpr int BYTES = 2 * HALF * 2;
  static_assert(2 * BYTES <= 160 * 1024, "two workgroups per CU");
};

// One quarter's operands (the thread's pieces: row e / 8, channels
// 4 (e % 8) .. + 3 of e = tid + NTHR u) from registers to LDS, split.
template <int DK, int QR, int QS>
__device__ __forceinline__ void b1_stage(bf16* sp, int tid, const f32x4 (&xr)[QR], const f32x4 (&xo)[QR],
                                         const f32x4 (&xw)[QR], const f32x4 (&xs)[QS], const f32x4 (&xd)[QS]) {
  using L = BwdB1Lay<DK>;
#pragma unroll
  for (int u = 0; u < QR; ++u) {
    const int e = tid + NTHR * u, r = e / (L::VH / 4), c4 = (e % (L::VH / 4)) * 4;
    put_split<L::SE>(sp, L::HALF, L::rR + r, c4, xr[u]);
    put_split<L::SE>(sp, L::HALF, L::rO + r, c4, xo[u]);
    put_split<L::SE>(sp, L::HALF, L::rW + r, c4, xw[u]);
  }
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    const int e = tid + NTHR * u, r = e / (L::VH / 4), c4 = (e % (L::VH / 4)) * 4;
    put_split<L::SE>(sp, L::HALF, L::rS + r, c4, xs[u]);
    put_split<L::SE>(sp, L::HALF, L::rdS + r, c4, xd[u]);
  }
}

// The products of row block w over one staged quarter:
//   dT += dR W^T, dA_qk += dO W^T (column blocks J <= w),
//   dE_bar += dR S^T, dQ_gamma += dO S^T, dK_tail += W dS^T
// (dT and dE_bar without their minus signs)
template <int DK>
__device__ __forceinline__ void b1_products(const bf16* sp, int w, int g, int l16, f32x4 (&aT)[4], f32x4 (&aA)[4],
                                            f32x4 (&aE)[DK / 16], f32x4 (&aQ)[DK / 16], f32x4 (&aK)[DK / 16]) {
  using L = BwdB1Lay<DK>;
  const bf16* base = sp + l16 * L::SE + 8 * g;
  auto frag = [&](int row0) __attribute__((always_inline)) { return lds_split(base + row0 * L::SE, L::HALF); };
  const SplitB ar = frag(L::rR + 16 * w), ao = frag(L::rO + 16 * w), aw = frag(L::rW + 16 * w);
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J > w) continue;  // wave-uniform
    const SplitB bw = frag(L::rW + 16 * J);
    aT[J] = mma_split(ar, bw, aT[J]);
    aA[J] = mma_split(ao, bw, aA[J]);
  }
#pragma unroll
  for (int c = 0; c < DK / 16; ++c) {
    const SplitB bs = frag(L::rS + 16 * c), bd = frag(L::rdS + 16 * c);
    aE[c] = mma_split(ar, bs, aE[c]);
    aQ[c] = mma_split(ao, bs, aQ[c]);
    aK[c] = mma_split(aw, bd, aK[c]);
  }
}

// the sum over 8 adjacent lanes (an aligned group), in every lane of it
__device__ __forceinline__ float sum8(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
  return x;
}

template <class IO, int DK, int DV>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_prod_kernel(BwdParams p) {
  using L = BwdB1Lay<DK>;
  constexpr int VH = L::VH, NC = DK / 16;
  constexpr int QR = CH * VH / 4 / NTHR, QS = DK * VH / 4 / NTHR;
  static_assert(DV % VH == 0, "value channels in quarters of 32");
  __shared__ __attribute__((aligned(16))) bf16 sp[2 * L::HALF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int N = p.nchunks;
  const size_t ch = blockIdx.x;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int bb = bh / p.f.H, hh = bh - bb * p.f.H;
  const int T = p.f.T, H = p.f.H;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* dog = reinterpret_cast<const IO*>(p.d_o);
  const BwdWs& ws = p.ws;

  f32x4 aT[4], aA[4], aE[NC], aQ[NC], aK[NC];
#pragma unroll
  for (int J = 0; J < 4; ++J) aT[J] = aA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) aE[c] = aQ[c] = aK[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sc[QS] = {};  // sum_v S (.) dS of the thread's pieces (key channel (tid + NTHR u) / 8)

  for (int vh = 0; vh < DV; vh += VH) {
    if (vh > 0) __syncthreads();  // the previous quarter's reads are done
    // ---- the quarter's rows to LDS (every load of the thread issued first)
    {
      f32x4 xr[QR], xo[QR], xw[QR], xs[QS], xd[QS];
#pragma unroll
      for (int u = 0; u < QR; ++u) {
        const int e = tid + NTHR * u, r = e / (VH / 4), c4 = (e % (VH / 4)) * 4;
        xr[u] = *reinterpret_cast<const f32x4*>(ws.dR + (ch * CH + r) * DV + vh + c4);
        xw[u] = *reinterpret_cast<const f32x4*>(ws.W + (ch * CH + r) * DV + vh + c4);
        xo[u] = ldf4(dog + (seq0 + (size_t)min(n * CH + r, T - 1) * H) * DV + vh + c4);
        if (n * CH + r >= T) xo[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < QS; ++u) {
        const int e = tid + NTHR * u, r = e / (VH / 4), c4 = (e % (VH / 4)) * 4;
        xs[u] = *reinterpret_cast<const f32x4*>(ws.S + (ch * DK + r) * DV + vh + c4);
        xd[u] = *reinterpret_cast<const f32x4*>(ws.dS + (ch * DK + r) * DV + vh + c4);
      }
      b1_stage<DK>(sp, tid, xr, xo, xw, xs, xd);
#pragma unroll
      for (int u = 0; u < QS; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[u] = __builtin_fmaf(xs[u][i], xd[u][i], sc[u]);
    }
    __syncthreads();
    b1_products<DK>(sp, w, g, l16, aT, aA, aE, aQ, aK);
  }
  // ---- outputs: lane holds rows 16 w + 4 g + r of column l16 of each block
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * g + r;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const int j = 16 * J + l16;
      const float t = J <= w && j < i ? -aT[J][r] : 0.f;   // dT: strictly lower
      const float a = J <= w && j <= i ? aA[J][r] : 0.f;   // dA_qk: lower
      ws.T[(ch * CH + i) * CH + j] = t;
      ws.A[(ch * CH + i) * CH + j] = a;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const size_t o = (ch * CH + i) * DK + 16 * c + l16;
      ws.Eb[o] = -aE[c][r];
      ws.Qg[o] = aQ[c][r];
      ws.Kt[o] = aK[c][r];
    }
  }
  // sC: a key channel's pieces lie in 8 adjacent lanes
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    const float s = sum8(sc[u]);
    if ((tid & 7) == 0) ws.gC[ch * DK + (tid + NTHR * u) / (VH / 4)] = s;
  }
}

// The end of pass B2, shared by both forms of it: the value side (dZ = dR
// gives dv and, per gate kind, dw or the write part of dbeta; each wave
// covers 64 columns of one row per step, every load issued first) and the
// per-token sums (the scalar-decay dg, dbeta, dlambda) from the rows' LDS
// partial sums.
template <class IO, int DK, int DV, int NPASS>
__device__ __forceinline__ void key_tail(const BwdParams& p, size_t ch, int t0, size_t seq0, int tid,
                                         const float* sBeta, float (*sRz)[DV / 64], const float* sDg,
                                         const float (*sRb)[NPASS], const float (*sRl)[NPASS]) {
  constexpr int VW = DV / 64;
  const int lane = tid & 63;
  const int T = p.f.T, H = p.f.H;
  const int decay = p.f.decay, erase = p.f.erase, write = p.f.write, qmix = p.f.qmix;
  const IO* vg = reinterpret_cast<const IO*>(p.f.v);
  const BwdWs& ws = p.ws;
  // (in groups of up to 16 elements per thread, every load of a group issued first)
  constexpr int NE = CH * DV / NTHR, UB = NE < 16 ? NE : 16;
  static_assert(NE % UB == 0, "whole groups");
#pragma unroll 1
  for (int u0 = 0; u0 < NE; u0 += UB) {
    const float* dz = ws.dR + ch * CH * DV;
    float zr[UB], vr[UB], wr[UB];
#pragma unroll
    for (int uu = 0; uu < UB; ++uu) {
      const int e = tid + NTHR * (u0 + uu), r = e / DV, v = e - r * DV;
      const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
      zr[uu] = dz[e];
      vr[uu] = ldf(vg + tok * DV + v);
      wr[uu] = write == 1 ? p.f.w[tok * DV + v] : 0.f;
    }
#pragma unroll
    for (int uu = 0; uu < UB; ++uu) {
      const int u = u0 + uu, e = tid + NTHR * u, r = e / DV, v = e - r * DV;
      const int t = t0 + r;
      const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
      const float z = zr[uu], vv = vr[uu];
      float zb = 0.f;
      if (t < T) {
        if (write == 1) {
          p.dw[tok * DV + v] = z * vv;
          p.dv[tok * DV + v] = wr[uu] * z;
        } else {
          zb = z * vv;
          p.dv[tok * DV + v] = sBeta[r] * z;
        }
      }
      zb = wave_total(zb);
      if (lane == 0) sRz[r][v >> 6] = zb;
    }
  }
  __syncthreads();
  // ---- per-token sums: the scalar-decay dg, dbeta, dlambda
  for (int r = tid; r < CH; r += NTHR) {
    const int t = t0 + r;
    if (t >= T) continue;
    const size_t tok = seq0 + (size_t)t * H;
    if (decay == 1) p.dg[tok] = sDg[r];
    float sb = 0.f, sl = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < NPASS; ++q2) {
      sb += sRb[r][q2];
      sl += sRl[r][q2];
    }
    if (write == 0) {
#pragma unroll
      for (int w2 = 0; w2 < VW; ++w2) sb += sRz[r][w2];
    }
    if (erase == 0 || write == 0) p.dbeta[tok] = sb;
    if (qmix == 2) p.dlam[tok] = sl;
    else if (qmix == 1) ws.dlam[tok] = sl;
  }
}

// ---- pass B2: back to the rows, the cumulative decay and the gates -----------
// Under a decay per key channel (this kernel) the weights d_ij[c] are formed
// per term.  The key channels are taken KC = 64 at a time, so that the
// chunk's k, e, q and G columns of the pass and the whole dT and dA_qk fit
// in LDS together; every inner-loop operand is then an LDS read (dT and
// dA_qk entries as broadcasts).  Thread (wave w, lane c) owns channel c of
// the pass in rows w, w + 4, ..., so each row of a pass is one wave and its
// sums over the channels are wave reductions.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(NTHR) void bwd_key_kernel(BwdParams p) {
  constexpr int KC = 64, NPASS = DK / KC;
  constexpr int NP = NTHR / KC, RPP = CH / NP;   // 4 row partitions of 16 rows
  constexpr int VW = DV / 64;                    // waves per row of the value side
  constexpr int TP = CH + 4;
  static_assert(DK % KC == 0, "key channels in passes of 64");
  __shared__ __attribute__((aligned(16))) float sK[CH * KC], sE[CH * KC], sQ[CH * KC], sG[CH * KC];
  __shared__ __attribute__((aligned(16))) float sdT[CH * TP], sdA[CH * TP];
  __shared__ float sGC[KC], sRb[CH][NPASS], sRl[CH][NPASS], sRz[CH][VW];
  __shared__ float sBeta[CH], sLam[CH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int N = p.nchunks;
  const size_t ch = blockIdx.x;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int bb = bh / p.f.H, hh = bh - bb * p.f.H;
  const int T = p.f.T, H = p.f.H;
  const int t0 = n * CH;
  const int erase = p.f.erase, qmix = p.f.qmix;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* qg = reinterpret_cast<const IO*>(p.f.q);
  const IO* kg = reinterpret_cast<const IO*>(p.f.k);
  const BwdWs& ws = p.ws;

  copy_rows<CH, CH, TP>(sdT, ws.T + ch * CH * CH, tid);
  copy_rows<CH, CH, TP>(sdA, ws.A + ch * CH * CH, tid);
  for (int r = tid; r < CH; r += NTHR) {
    const int t = t0 + r;
    const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
    sBeta[r] = (t < T && (erase == 0 || p.f.write == 0)) ? p.f.beta[tok] : 0.f;
    sLam[r] = (t < T && qmix) ? (qmix == 2 ? p.f.lam[tok] : p.f.lam[hh]) : 0.f;
  }
  const int c = lane;
  const int par = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int ps = 0; ps < NPASS; ++ps) {
    const int cg = ps * KC + c;  // key channel of this thread
    __syncthreads();             // the previous pass's columns are no longer read
    // ---- this pass's columns of the chunk's rows (zero past T)
    {
      constexpr int QPR = KC / 4, NQ = CH * QPR / NTHR;
      f32x4 rk[NQ], rq[NQ], rg[NQ], rb[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int e = tid + NTHR * u, r = e / QPR, c4 = ps * KC + (e - r * QPR) * 4;
        const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
        rk[u] = ldf4(kg + tok * DK + c4);
        rq[u] = ldf4(qg + tok * DK + c4);
        rg[u] = ldf4(p.f.g + tok * DK + c4);
        if (erase == 1) rb[u] = ldf4(p.f.b + tok * DK + c4);
      }
      __syncthreads();  // sBeta, sLam
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int e = tid + NTHR * u, r = e / QPR, cl = (e - r * QPR) * 4;
        const bool ok = t0 + r < T;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float kv = ok ? rk[u][i] : 0.f, qv = ok ? rq[u][i] : 0.f;
          sK[r * KC + cl + i] = kv;
          sQ[r * KC + cl + i] = qv;
          sE[r * KC + cl + i] = erase == 1 ? (ok ? rb[u][i] : 0.f) * kv
                                           : sBeta[r] * __builtin_fmaf(sLam[r], qv, kv);
          sG[r * KC + cl + i] = ok ? rg[u][i] : 0.f;
        }
      }
    }
    __syncthreads();
    if (tid < KC) {
      float run = 0.f;
      for (int r = 0; r < CH; ++r) {
        run += sG[r * KC + tid];
        sG[r * KC + tid] = run;
      }
      sGC[tid] = run;
    }
    // the product pass's results for my rows
    float dEb[RPP], dQg[RPP], dKt[RPP], bI[RPP];
#pragma unroll
    for (int m = 0; m < RPP; ++m) {
      const int i = par + NP * m;
      const size_t at = (ch * CH + i) * DK + cg;
      dEb[m] = ws.Eb[at];
      dQg[m] = ws.Qg[at];
      dKt[m] = ws.Kt[at];
      const int t = t0 + i;
      bI[m] = (erase == 1 && t < T) ? p.f.b[(seq0 + (size_t)t * H) * DK + cg] : 0.f;
    }
    __syncthreads();
    const float GC = sGC[c];
    float dGr[RPP], xkt[RPP];
#pragma unroll
    for (int m = 0; m < RPP; ++m) {
      const int i = par + NP * m;  // wave-uniform
      const float gi = sG[i * KC + c];
      const float gam = fexp(gi), tl = fexp(GC - gi);
      const float ki = sK[i * KC + c], ei = sE[i * KC + c], qi = sQ[i * KC + c];
      // off-diagonal sums (the diagonal of A_qk has d_ii = 1 and does not
      // depend on G: its two contributions to dG cancel exactly, so it is
      // kept out of dG rather than added and cancelled in fp32)
      float P = 0.f, Pq = 0.f, Rm = 0.f, Rq = 0.f;
      for (int j = 0; j < i; ++j) {
        const float kd = sK[j * KC + c] * fexp(gi - sG[j * KC + c]);
        P = __builtin_fmaf(sdT[i * TP + j], kd, P);
        Pq = __builtin_fmaf(sdA[i * TP + j], kd, Pq);
      }
      for (int i2 = i + 1; i2 < CH; ++i2) {
        const float d = fexp(sG[i2 * KC + c] - gi);
        Rm = __builtin_fmaf(sdT[i2 * TP + i], sE[i2 * KC + c] * d, Rm);
        Rq = __builtin_fmaf(sdA[i2 * TP + i], sQ[i2 * KC + c] * d, Rq);
      }
      const float diag = sdA[i * TP + i];
      const float de = __builtin_fmaf(gam, dEb[m], P);
      float dqd = __builtin_fmaf(gam, dQg[m], __builtin_fmaf(diag, ki, Pq));
      float dkd = tl * dKt[m] + Rm + __builtin_fmaf(diag, qi, Rq);
      dGr[m] = ei * gam * dEb[m] + qi * gam * dQg[m] + ei * P + qi * Pq - ki * (Rm + Rq);
      xkt[m] = ki * tl * dKt[m];  // K_tail_i dK_tail_i
      // the erase gate
      float rb = 0.f, rl = 0.f;
      const int t = t0 + i;
      const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
      if (erase == 1) {
        if (t < T) p.db[tok * DK + cg] = de * ki;
        dkd = __builtin_fmaf(bI[m], de, dkd);
      } else {
        const float bt = sBeta[i], lt = sLam[i];
        rb = de * __builtin_fmaf(lt, qi, ki);
        dkd = __builtin_fmaf(bt, de, dkd);
        if (qmix) {
          dqd = __builtin_fmaf(bt * lt, de, dqd);
          rl = bt * de * qi;
        }
      }
      if (t < T) {
        p.dq[tok * DK + cg] = dqd;
        p.dk[tok * DK + cg] = dkd;
      }
      rb = wave_total(rb);
      rl = wave_total(rl);
      if (lane == 0) {
        sRb[i][ps] = rb;
        sRl[i][ps] = rl;
      }
    }
    __syncthreads();  // sG takes dG, sE the K_tail terms
#pragma unroll
    for (int m = 0; m < RPP; ++m) {
      const int i = par + NP * m;
      sG[i * KC + c] = dGr[m];
      sE[i * KC + c] = xkt[m];
    }
    __syncthreads();
    // dg_t = sum_{r>=t} dG_r + sum_{j<t} K_tail_j dK_tail_j + gamma_C sC
    if (tid < KC) {
      float pre = 0.f;
      for (int r = 0; r < CH; ++r) {  // exclusive prefix of the K_tail terms
        const float x = sE[r * KC + tid];
        sE[r * KC + tid] = pre;
        pre += x;
      }
      const float base = fexp(GC) * ws.gC[ch * DK + ps * KC + tid];
      float run = 0.f;
      for (int r = CH - 1; r >= 0; --r) {
        run += sG[r * KC + tid];
        const float dgv = run + sE[r * KC + tid] + base;
        if (t0 + r < T) p.dg[(seq0 + (size_t)(t0 + r) * H) * DK + ps * KC + tid] = dgv;
      }
    }
  }
  key_tail<IO, DK, DV, NPASS>(p, ch, t0, seq0, tid, sBeta, sRz, nullptr, sRb, sRl);
}

// ---- passes B1 and B2 in one kernel, under a scalar decay (or none) ---------
// One workgroup of four waves per (batch, head, chunk), two per CU.  Phase 1
// is the product pass (bwd_prod_kernel's quarters of 32 value channels),
// together with the value side (dv, dw, and the rows' sums of dZ (.) v);
// phase 2 is the key pass under a scalar decay in passes of 32 key channels,
// as bwd_key_scalar_kernel would run it, but dT and dA_qk go from phase 1's
// accumulators straight to LDS as D1 = dT (.) D and D2 = dA_qk (.) D, and
// dE_bar, dQ_gamma, dK_tail stay in the accumulators: the lane that holds
// row 16 w + 4 g + r of column 16 c + l of dE_bar after phase 1 is the lane
// that needs it in phase 2.  None of the five products goes to the workspace
// and comes back (256 KB per chunk at dk = dv = 128).  Phase 2's arrays
// overlay phase 1's.
template <int DK>
struct BwdPKLay {
  static constexpr int P1 = BwdB1Lay<DK>::BYTES / 4;  // phase 1: a quarter's split rows (floats)
  static constexpr int KC = 32, TP = CH + 4;  // phase 2: D1, D2 and a pass's K^T, E^T, Q^T
  static constexpr int oD1 = 0, oD2 = oD1 + CH * TP, oKT = oD2 + CH * TP, oET = oKT + KC * TP, oQT = oET + KC * TP;
  static constexpr int P2 = oQT + KC * TP;
  static constexpr int TOTAL = P1 > P2 ? P1 : P2;
  static constexpr int SMALL = (2 * CH * (DK / KC) + 8 * CH + DK) * 4;  // the per-row and per-channel arrays
  static_assert(2 * (TOTAL * 4 + SMALL) <= 160 * 1024, "two workgroups per CU");
};

template <class IO, int DK, int DV>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_prodkey_kernel(BwdParams p) {
  using L = BwdPKLay<DK>;
  constexpr int VH = BwdB1Lay<DK>::VH, NC = DK / 16;
  constexpr int KC = L::KC, TP = L::TP, NPASS = DK / KC, NCB = KC / 16;
  static_assert(DV % VH == 0 && DK % KC == 0 && NTHR == 256, "quarters of 32 value channels, passes of 32 key channels");
  __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
  __shared__ float sRb[CH][NPASS], sRl[CH][NPASS], sRz[CH], sDg[CH], sSC[DK];
  __shared__ float sBeta[CH], sLam[CH], sGt[CH], sDiag[CH], sRG[CH], sRX[CH];
  bf16* sp = reinterpret_cast<bf16*>(lds);
  float *sD1 = lds + L::oD1, *sD2 = lds + L::oD2, *sKT = lds + L::oKT, *sET = lds + L::oET, *sQT = lds + L::oQT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int N = p.nchunks;
  const size_t ch = blockIdx.x;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int bb = bh / p.f.H, hh = bh - bb * p.f.H;
  const int T = p.f.T, H = p.f.H;
  const int t0 = n * CH;
  const int decay = p.f.decay, erase = p.f.erase, write = p.f.write, qmix = p.f.qmix;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* qg = reinterpret_cast<const IO*>(p.f.q);
  const IO* kg = reinterpret_cast<const IO*>(p.f.k);
  const IO* vg = reinterpret_cast<const IO*>(p.f.v);
  const IO* dog = reinterpret_cast<const IO*>(p.d_o);
  const BwdWs& ws = p.ws;

  for (int r = tid; r < CH; r += NTHR) {
    const int t = t0 + r;
    const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
    sBeta[r] = (t < T && (erase == 0 || write == 0)) ? p.f.beta[tok] : 0.f;
    sLam[r] = (t < T && qmix) ? (qmix == 2 ? p.f.lam[tok] : p.f.lam[hh]) : 0.f;
    sDg[r] = 0.f;
    sRG[r] = 0.f;
    sRX[r] = 0.f;
  }
  // the scalar decay's prefix sums G_t (zero past T)
  if (tid < CH) {
    const int t = t0 + tid;
    const float gv = (decay == 1 && t < T) ? p.f.g[seq0 + (size_t)t * H] : 0.f;
    sGt[tid] = wave_incl_scan(gv);
  }

  // ================= phase 1: the products over the value channels ==========
  // bwd_prod_kernel's quarters (b1_stage, b1_products: split precision).
  // The value side takes the thread's dR pieces of the quarter (row r,
  // channels c4 .. + 3) from its staging registers.
  constexpr int QR = CH * VH / 4 / NTHR, QS = DK * VH / 4 / NTHR;
  f32x4 aT[4], aA[4], aE[NC], aQ[NC], aK[NC];
#pragma unroll
  for (int J = 0; J < 4; ++J) aT[J] = aA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) aE[c] = aQ[c] = aK[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sc[QS] = {};       // sum_v S (.) dS of the thread's pieces (key channel (tid + NTHR u) / 8)
  float zrow[QR] = {};     // sum_v dZ (.) v of the thread's pieces (the beta write gate)
  for (int vh = 0; vh < DV; vh += VH) {
    if (vh > 0) __syncthreads();  // the previous quarter's reads are done
    f32x4 xr[QR], xo[QR], xw[QR], xs[QS], xd[QS], wv[QR];
    typename Raw<IO>::v4 vv[QR];
#pragma unroll
    for (int u = 0; u < QR; ++u) {
      const int e = tid + NTHR * u, r = e / (VH / 4), c4 = (e % (VH / 4)) * 4;
      const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
      xr[u] = *reinterpret_cast<const f32x4*>(ws.dR + (ch * CH + r) * DV + vh + c4);
      xw[u] = *reinterpret_cast<const f32x4*>(ws.W + (ch * CH + r) * DV + vh + c4);
      xo[u] = ldf4(dog + tok * DV + vh + c4);
      vv[u] = ldraw4(vg + tok * DV + vh + c4);
      if (write == 1) wv[u] = *reinterpret_cast<const f32x4*>(p.f.w + tok * DV + vh + c4);
    }
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      const int e = tid + NTHR * u, r = e / (VH / 4), c4 = (e % (VH / 4)) * 4;
      xs[u] = *reinterpret_cast<const f32x4*>(ws.S + (ch * DK + r) * DV + vh + c4);
      xd[u] = *reinterpret_cast<const f32x4*>(ws.dS + (ch * DK + r) * DV + vh + c4);
    }
#pragma unroll
    for (int u = 0; u < QR; ++u) {
      const int r = (tid + NTHR * u) / (VH / 4);
      if (t0 + r >= T) xo[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    b1_stage<DK>(sp, tid, xr, xo, xw, xs, xd);
#pragma unroll
    for (int u = 0; u < QS; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[u] = __builtin_fmaf(xs[u][i], xd[u][i], sc[u]);
    __syncthreads();  // (also: the per-row scalars are in place)
    // ---- the value side: dZ = dR gives dv and, per write gate, dw or the
    // rows' sums for dbeta
#pragma unroll
    for (int u = 0; u < QR; ++u) {
      const int e = tid + NTHR * u, r = e / (VH / 4), c4 = (e % (VH / 4)) * 4;
      const int t = t0 + r;
      if (t < T) {
        const size_t o = (seq0 + (size_t)t * H) * DV + vh + c4;
        const f32x4 z = xr[u], v4 = widen(vv[u]);
        if (write == 1) {
          *reinterpret_cast<f32x4*>(p.dw + o) = z * v4;
          *reinterpret_cast<f32x4*>(p.dv + o) = wv[u] * z;
        } else {
          zrow[u] += z[0] * v4[0] + z[1] * v4[1] + z[2] * v4[2] + z[3] * v4[3];
          *reinterpret_cast<f32x4*>(p.dv + o) = sBeta[r] * z;
        }
      }
    }
    b1_products<DK>(sp, w, g, l16, aT, aA, aE, aQ, aK);
  }
  // the rows' sums of dZ (.) v: a row's 32 channels of a quarter lie in 8
  // adjacent lanes
#pragma unroll
  for (int u = 0; u < QR; ++u) {
    const float z = sum8(zrow[u]);
    if ((tid & 7) == 0) sRz[(tid + NTHR * u) / (VH / 4)] = z;
  }
  // sC: a key channel's pieces lie in 8 adjacent lanes
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    const float z = sum8(sc[u]);
    if ((tid & 7) == 0) sSC[(tid + NTHR * u) / (VH / 4)] = z;
  }
  __syncthreads();  // phase 1's arrays are no longer read

  // ================= phase 2: back to the rows =================
  // D1, D2 strictly below the diagonal (the diagonal of dA_qk kept apart),
  // from this wave's blocks J <= w; the blocks above are never read
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J > w) continue;  // wave-uniform
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * w + 4 * g + r, j = 16 * J + l16;
      const float d = j < i ? fexp(sGt[i] - sGt[j]) : 0.f;
      sD1[i * TP + j] = -aT[J][r] * d;
      sD2[i * TP + j] = aA[J][r] * d;
      if (j == i) sDiag[i] = aA[J][r];
    }
  }
  const float GC = sGt[CH - 1];
  // a row's sum over the 16 lanes of its group (quad permutations, then the
  // half-row and row mirrors)
  auto row16 = [](float x) __attribute__((always_inline)) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xf, 0xf, true));
    return x;
  };

#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    // ps = 0: D1, D2 and the diagonal are in place; later: the previous
    // pass's columns are no longer read
    __syncthreads();
    // ---- this pass's columns of the chunk's rows, transposed (zero past T):
    // lane (h, k, j) = (lane / 32, lane / 4 % 8, lane % 4) of wave w takes
    // token 4 b + j (b = 2 (w + 4 u) + h), channels 4 k .. + 3 of the pass;
    // the quad transposes its block, and the lane writes channel 4 k + j,
    // tokens 4 b .. + 3 as one 16-byte LDS write
    {
      constexpr int NQ = CH * KC / 4 / NTHR;
      const int qj = lane & 3, cq = (lane >> 2) & 7, th = lane >> 5;
      f32x4 rk[NQ], rq[NQ], rb[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int r = 4 * (2 * (w + 4 * u) + th) + qj;
        const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
        rk[u] = ldf4(kg + tok * DK + ps * KC + 4 * cq);
        rq[u] = ldf4(qg + tok * DK + ps * KC + 4 * cq);
        if (erase == 1) rb[u] = ldf4(p.f.b + tok * DK + ps * KC + 4 * cq);
      }
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int b4 = 2 * (w + 4 * u) + th, r = 4 * b4 + qj;
        const bool ok = t0 + r < T;
        f32x4 kv, qv, ev;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kv[i] = ok ? rk[u][i] : 0.f;
          qv[i] = ok ? rq[u][i] : 0.f;
          ev[i] = erase == 1 ? (ok ? rb[u][i] : 0.f) * kv[i] : sBeta[r] * __builtin_fmaf(sLam[r], qv[i], kv[i]);
        }
        const int c = 4 * cq + qj;
        *reinterpret_cast<f32x4*>(sKT + c * TP + 4 * b4) = quad_transpose(kv, qj);
        *reinterpret_cast<f32x4*>(sQT + c * TP + 4 * b4) = quad_transpose(qv, qj);
        *reinterpret_cast<f32x4*>(sET + c * TP + 4 * b4) = quad_transpose(ev, qj);
      }
    }
    // the erase gate at my (row, channel) pairs, requested before the products
    float bI[NCB][4];
#pragma unroll
    for (int C = 0; C < NCB; ++C)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * w + 4 * g + r, cg = ps * KC + 16 * C + l16;
        bI[C][r] = (erase == 1 && t < T) ? p.f.b[(seq0 + (size_t)t * H) * DK + cg] : 0.f;
      }
    __syncthreads();
    // ---- the four products: row block w, column blocks C of the pass
    f32x4 aP[NCB], aPq[NCB], aRm[NCB], aRq[NCB];
#pragma unroll
    for (int C = 0; C < NCB; ++C) aP[C] = aPq[C] = aRm[C] = aRq[C] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J <= w) {  // P, Pq: j < i
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(sD1 + (16 * w + l16) * TP + 16 * J + 4 * g);
        const f32x4 a2 = *reinterpret_cast<const f32x4*>(sD2 + (16 * w + l16) * TP + 16 * J + 4 * g);
#pragma unroll
        for (int C = 0; C < NCB; ++C) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(sKT + (16 * C + l16) * TP + 16 * J + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            aP[C] = mfma_f32(a1[r], b[r], aP[C]);
            aPq[C] = mfma_f32(a2[r], b[r], aPq[C]);
          }
        }
      }
      if (J >= w) {  // Rm, Rq: i2 > i; column 16 w + l16 of D1, D2 at rows 16 J + 4 g + r
        float a1[4], a2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a1[r] = sD1[(16 * J + 4 * g + r) * TP + 16 * w + l16];
          a2[r] = sD2[(16 * J + 4 * g + r) * TP + 16 * w + l16];
        }
#pragma unroll
        for (int C = 0; C < NCB; ++C) {
          const f32x4 be = *reinterpret_cast<const f32x4*>(sET + (16 * C + l16) * TP + 16 * J + 4 * g);
          const f32x4 bq = *reinterpret_cast<const f32x4*>(sQT + (16 * C + l16) * TP + 16 * J + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            aRm[C] = mfma_f32(a1[r], be[r], aRm[C]);
            aRq[C] = mfma_f32(a2[r], bq[r], aRq[C]);
          }
        }
      }
    }
    // ---- rows: the gradients of q, k and e, the erase gate, the row sums
    float gam[4], tl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gi = sGt[16 * w + 4 * g + r];
      gam[r] = fexp(gi);
      tl[r] = fexp(GC - gi);
    }
    float sb[4] = {0.f, 0.f, 0.f, 0.f}, sl[4] = {0.f, 0.f, 0.f, 0.f};
    float sg[4] = {0.f, 0.f, 0.f, 0.f}, sx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int C = 0; C < NCB; ++C) {
      const int c = 16 * C + l16, cg = ps * KC + c, cb = NCB * ps + C;  // cb: column block of phase 1
      const f32x4 kv = *reinterpret_cast<const f32x4*>(sKT + c * TP + 16 * w + 4 * g);
      const f32x4 ev = *reinterpret_cast<const f32x4*>(sET + c * TP + 16 * w + 4 * g);
      const f32x4 qv = *reinterpret_cast<const f32x4*>(sQT + c * TP + 16 * w + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * g + r;
        const float ki = kv[r], ei = ev[r], qi = qv[r];
        const float dEb = -aE[cb][r], dQg = aQ[cb][r], dKt = aK[cb][r];
        const float P = aP[C][r], Pq = aPq[C][r], Rm = aRm[C][r], Rq = aRq[C][r];
        const float diag = sDiag[i];
        const float de = __builtin_fmaf(gam[r], dEb, P);
        float dqd = __builtin_fmaf(gam[r], dQg, __builtin_fmaf(diag, ki, Pq));
        float dkd = tl[r] * dKt + Rm + __builtin_fmaf(diag, qi, Rq);
        // (the diagonal of A_qk stays out of dG: its two terms cancel exactly)
        sg[r] += ei * gam[r] * dEb + qi * gam[r] * dQg + ei * P + qi * Pq - ki * (Rm + Rq);
        sx[r] += ki * tl[r] * dKt;  // K_tail_i dK_tail_i
        const int t = t0 + i;
        const size_t tok = seq0 + (size_t)min(t, T - 1) * H;
        if (erase == 1) {
          if (t < T) p.db[tok * DK + cg] = de * ki;
          dkd = __builtin_fmaf(bI[C][r], de, dkd);
        } else {
          const float bt = sBeta[i], lt = sLam[i];
          sb[r] += de * __builtin_fmaf(lt, qi, ki);
          dkd = __builtin_fmaf(bt, de, dkd);
          if (qmix) {
            dqd = __builtin_fmaf(bt * lt, de, dqd);
            sl[r] += bt * de * qi;
          }
        }
        if (t < T) {
          p.dq[tok * DK + cg] = dqd;
          p.dk[tok * DK + cg] = dkd;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rb = row16(sb[r]), rl = row16(sl[r]), rg = row16(sg[r]), rx = row16(sx[r]);
      if (l16 == 0) {
        const int i = 16 * w + 4 * g + r;
        sRb[i][ps] = rb;
        sRl[i][ps] = rl;
        sRG[i] += rg;  // (one writer per row; the passes are ordered by barriers)
        sRX[i] += rx;
      }
    }
  }
  __syncthreads();
  // dg_t = sum_{r>=t} RG_r + sum_{j<t} RX_j + gamma_C sum_c sC[c] (the
  // per-channel form summed over the channels), by wave prefix sums
  if (decay == 1 && tid < CH) {
    float s2 = 0.f;
    for (int c2 = tid; c2 < DK; c2 += CH) s2 += sSC[c2];
    const float base = fexp(GC) * wave_total(s2);
    // a true exclusive prefix and a true suffix (scan of the reversed rows):
    // a total minus a prefix would add a row's term and take it away again,
    // and the O(1) K_tail term of the last row (tail = 1) would leave its
    // rounding in every other token's dg, which under a strong decay is
    // orders of magnitude smaller
    const float rx = sRX[tid];
    const float ix = wave_incl_scan(rx), ixm = __shfl_up(ix, 1);
    const float ex = lane == 0 ? 0.f : ixm;
    const float sg = __shfl(wave_incl_scan(__shfl(sRG[tid], 63 - lane)), 63 - lane);
    sDg[tid] = sg + ex + base;
  }
  __syncthreads();
  // ---- per-token sums: the scalar-decay dg, dbeta, dlambda
  for (int r = tid; r < CH; r += NTHR) {
    const int t = t0 + r;
    if (t >= T) continue;
    const size_t tok = seq0 + (size_t)t * H;
    if (decay == 1) p.dg[tok] = sDg[r];
    float sb = 0.f, sl = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < NPASS; ++q2) {
      sb += sRb[r][q2];
      sl += sRl[r][q2];
    }
    if (write == 0) sb += sRz[r];
    if (erase == 0 || write == 0) p.dbeta[tok] = sb;
    if (qmix == 2) p.dlam[tok] = sl;
    else if (qmix == 1) ws.dlam[tok] = sl;
  }
}

// ---- a per-head lambda: the sum of its per-token gradients ------------------
__global__ __launch_bounds__(256) void bwd_lam_reduce_kernel(const float* dlam_t, float* dlam, int B, int T,
                                                             int H) {
  __shared__ float part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int64_t n = (int64_t)B * T;
  float s = 0.f;
  for (int64_t i = tid; i < n; i += 256) s += dlam_t[i * H + h];
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) dlam[h] = part[0];
}

}  // namespace gdr
