// Chunkwise forward of the generalized gated delta rule on gfx950.
//
// Algorithm: the chunk WY form with absorbed decay of "Gated DeltaNet-2:
// Decoupling Erase and Write in Linear Attention" (key design 2).  Per chunk
// of C = 64 tokens and state S_[n] entering it:
//   G_r = chunk-local inclusive cumsum of g, gamma_r = exp(G_r)
//   T    = tril(E_bar K_bar^T, -1),  A = (I + T)^{-1}      (e_bar = gamma e, k_bar = k / gamma)
//   Y    = A E_bar,  U = A Z
//   W    = U - Y S_[n]
//   O    = Q_gamma S_[n] + A_qk W,  A_qk = tril(Q_gamma K_bar^T, 0)
//   S_[n+1] = Diag(gamma_C) S_[n] + K_tail^T W,  K_tail[j] = (gamma_C / gamma_j) k_j
// (the page leaves Q_gamma, A_qk, K_tail implicit; they follow from writing
// the post-update readout with S_r = Diag(gamma_r) S^_r).
//
// The page's k_bar = gamma^{-1} k is never formed: at per-channel decays
// gamma^{-1} leaves the fp32 range within a chunk.  The entries
//   T[i][j] = sum_c e_i[c] k_j[c] exp(G_i[c] - G_j[c])
// are formed instead as products of bounded factors (see gram_channel).
//
// One workgroup (4 waves) owns one (batch, head) and a slice of DVS value
// columns, keeps that slice of the fp32 state in MFMA accumulators for the
// whole sequence and walks the chunks in order.  Each chunk:
//   prep    load q, k, v, gates (prefetched one chunk ahead); cumulative
//           log-decay; write the MFMA operands to LDS
//   gram    T and A_qk (MFMA)
//   solve   A = (I + T)^{-1}: 16x16 diagonal blocks by forward substitution
//           on the vector ALUs, then two levels of block combination (MFMA)
//   wy      Y^T = E_bar^T A^T, U = A Z (MFMA); S^T to LDS
//   state   W = U - Y S, O^T = S^T Q_gamma^T + W^T A_qk^T, S += K_tail^T W
#pragma once

#include "common.hpp"

namespace gdr {

constexpr int CH = 64;     // chunk length C
constexpr int NTHR = 256;  // threads per workgroup (4 waves)

struct ChunkParams {
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
  int B, T, H, DV;
  int decay;  // 0 none, 1 scalar, 2 channel
  int erase;  // 0 beta, 1 channel
  int write;  // 0 beta, 1 channel
  int qmix;
  int nslices;
  const void* ws;  // workspace records of the two-pass forms (else unused)
};

// largest 16-token log-decay window for which the bounded-factor Gram is
// used; exp(80) * |k| stays finite in bf16/fp32 with margin
constexpr float WINDOW_LIMIT = 80.f;

// ---- LDS layout (byte offsets) -------------------------------------------
template <class CT, int DK, int DVS, bool CHAN>
struct Lay {
  static constexpr int E = sizeof(CT);
  static constexpr int PAD = 16 / E;
  static constexpr int SK = DK + PAD;  // row stride of [rows][DK] arrays
  static constexpr int SC = CH + PAD;  // row stride of [rows][64] arrays
  static constexpr int SP = 16 + PAD;  // solve scratch, level 1
  static constexpr int SP2 = 32 + PAD; // solve scratch, level 2
  static constexpr int TDS = 20;       // diagonal T blocks, fp32 row stride
  static constexpr bool CM = (E == 2); // bf16 fragments need a column-major copy of A
  static constexpr int FBC = 8;        // channels per fallback slab
  static constexpr int FBS = FBC + 1;  // fallback slab row stride (floats)
  static constexpr int CG = DK / 8;
  static constexpr int TG = NTHR / CG;

  // persistent through the chunk
  static constexpr int oQ = 0;                            // [64][SK]  q (scalar) / Q_gamma (channel)
  static constexpr int oEbT = oQ + CH * SK * E;           // [DK][SC]  E_bar^T
  static constexpr int oKtT = oEbT + DK * SC * E;         // [DK][SC]  K_tail^T
  static constexpr int oZT = oKtT + DK * SC * E;          // [DVS][SC] Z^T
  static constexpr int oArm = oZT + DVS * SC * E;         // [64][SC]  A, row-major
  static constexpr int oAcm = oArm + CH * SC * E;         // [64][SC]  A, column-major (bf16)
  static constexpr int oAqk = oAcm + (CM ? CH * SC * E : 0);  // [64][SC] A_qk row-major
  static constexpr int oP = oAqk + CH * SC * E;           // solve scratch 2 x [16][SP2]
  static constexpr int oG = oP + 2 * 16 * SP2 * E;        // 64 floats: chunk cumsum (scalar decay)
  static constexpr int oBeta = oG + 256;                  // 64 floats
  static constexpr int oGam = oBeta + 256;                // 64 floats: gamma (scalar decay)
  static constexpr int oGamC = oGam + 256;                // DK floats: gamma_C per channel
  static constexpr int oGs = oGamC + DK * 4;              // [4][DK] floats: G at the 16-block starts
  static constexpr int oFlag = oGs + 4 * DK * 4;          // int: fallback flag
  static constexpr int oR1 = oFlag + 16;
  // union region R1, phase 1 (prep / gram / solve)
  static constexpr int oK = oR1;                          // scalar: [64][SK] K;  channel: [64][SK] K-side factors
  static constexpr int oEb = oK + CH * SK * E;            // scalar: [64][SK] erase base; channel: Xe [16][SK], Xq [16][SK]
  static constexpr int szOps = CHAN ? (CH + 32) * SK * E : 2 * CH * SK * E;
  static constexpr int oTd = oR1 + szOps;                 // [4][16][TDS] fp32 diagonal blocks of T
  static constexpr int oTb = oTd + 4 * 16 * TDS * 4;      // [64][SC] T row-major
  static constexpr int endGram = oTb + CH * SC * E;
  static constexpr int oFB = endGram;                     // channel fallback: 4 x [64][FBS] fp32
  static constexpr int endFB = oFB + (CHAN ? 4 * CH * FBS * 4 : 0);
  static constexpr int endScan = oR1 + (CHAN ? TG * DK * 4 : 0);  // channel prep scan [TG][DK] fp32
  // union region R1, phase 2 (after the solve)
  static constexpr int oY = oR1;                          // [64][SK]  -Y
  static constexpr int oST = oY + CH * SK * E;            // [DVS][SK] S^T
  static constexpr int oWT = oST + DVS * SK * E;          // [DVS][SC] W^T
  static constexpr int endPost = oWT + DVS * SC * E;

  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int TOTAL = cmax(cmax(endFB, endPost), endScan);
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
  static_assert(oP % 16 == 0 && oR1 % 16 == 0 && oTb % 16 == 0 && oST % 16 == 0 && oWT % 16 == 0,
                "alignment");
};

// Lower block pair p (0..9) of the 4x4 grid of 16x16 blocks, row-major over
// I >= J: p = I (I + 1) / 2 + J.
__device__ __forceinline__ int pair_I(int p) { return p >= 6 ? 3 : (p >= 3 ? 2 : (p >= 1 ? 1 : 0)); }
__device__ __forceinline__ int pair_J(int p) { return p - (pair_I(p) * (pair_I(p) + 1)) / 2; }

// "Row tiles": the 4 x NV tiles (I = 16-token block, n = 16-column value
// block) of U, W and O^T, NV per wave.  With 4 value blocks each wave owns a
// value block; otherwise waves split the token blocks.
template <int NV>
__device__ __forceinline__ int rt_I(int t, int wave) {
  if constexpr (NV == 4) return t;
  else if constexpr (NV == 2) return (wave >> 1) + 2 * t;
  else return wave;
}
template <int NV>
__device__ __forceinline__ int rt_N(int t, int wave) {
  if constexpr (NV == 4) return wave;
  else if constexpr (NV == 2) return wave & 1;
  else return 0;
}

// Gate modes (erase kind, write kind): 0 = (BETA, BETA), 1 = (CHANNEL, CHANNEL),
// 2 = (CHANNEL, BETA), 3 = (BETA, CHANNEL).  Compile-time, so that every
// global load in the chunk loop is unconditional and can be issued a chunk
// ahead of its use.
template <int GM> struct Gates {
  static constexpr bool ERASE_CH = (GM == 1 || GM == 2);
  static constexpr bool WRITE_CH = (GM == 1 || GM == 3);
  static constexpr bool NEED_BETA = !ERASE_CH || !WRITE_CH;
};

template <class IO, class CT, int DK, int DVS, bool CHAN, int GM>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_fwd_kernel(ChunkParams p) {
  using L = Lay<CT, DK, DVS, CHAN>;
  constexpr int SK = L::SK, SC = L::SC, SP = L::SP, SP2 = L::SP2, TDS = L::TDS;
  constexpr int MC = DK / 64;   // 16-row state blocks per wave
  constexpr int NV = DVS / 16;  // 16-column value blocks
  constexpr int CG = L::CG, TG = L::TG, TPT = CH / TG;
  constexpr int VG = DVS / 8, VTG = NTHR / VG, VPT = (CH + VTG - 1) / VTG;
  static_assert(TPT == 2 || TPT == 4, "prep layout");
  static_assert(VPT == 1 || VPT == 2, "v layout");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (batch, head, value slice); the slices of one head get
  // consecutive indices after the remap, and blockIdx values that share a
  // residue mod 8 run on the same XCD, so they share its L2.
  int wid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) wid = (wid & 7) * (nwg >> 3) + (wid >> 3);
  const int NS = p.nslices;
  const int bh = wid / NS, slice = wid - bh * NS;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H, DV = p.DV;
  const int vbase = slice * DVS;
  const int nchunks = (T + CH - 1) / CH;
  const bool has_decay = p.decay != 0;
  constexpr bool erase_ch = Gates<GM>::ERASE_CH, write_ch = Gates<GM>::WRITE_CH;
  constexpr bool need_beta = Gates<GM>::NEED_BETA;
  const bool qmix = p.qmix != 0;
  const float lam = qmix ? p.lam[hh] : 0.f;

  // per-sequence base pointers; offsets inside one sequence are 32-bit
  // (the host checks T * H * max(dk, dv) < 2^31)
  const size_t seq0 = (size_t)bb * T * H + hh;  // token index of (bb, t = 0, hh)
  const IO* qg = reinterpret_cast<const IO*>(p.q) + seq0 * DK;
  const IO* kg = reinterpret_cast<const IO*>(p.k) + seq0 * DK;
  const IO* vg_ = reinterpret_cast<const IO*>(p.v) + seq0 * DV + vbase;
  IO* og = reinterpret_cast<IO*>(p.o) + seq0 * DV + vbase;
  const float* g_seq = p.g ? p.g + seq0 * (CHAN ? DK : 1) : nullptr;
  const float* beta_seq = p.beta ? p.beta + seq0 : nullptr;
  const float* b_seq = p.b ? p.b + seq0 * DK : nullptr;
  const float* w_seq = p.w ? p.w + seq0 * DV + vbase : nullptr;

  CT* sQ = reinterpret_cast<CT*>(smem + L::oQ);
  CT* sEbT = reinterpret_cast<CT*>(smem + L::oEbT);
  CT* sKtT = reinterpret_cast<CT*>(smem + L::oKtT);
  CT* sZT = reinterpret_cast<CT*>(smem + L::oZT);
  CT* sArm = reinterpret_cast<CT*>(smem + L::oArm);
  CT* sAcm = reinterpret_cast<CT*>(smem + L::oAcm);
  CT* sAqk = reinterpret_cast<CT*>(smem + L::oAqk);
  CT* sP = reinterpret_cast<CT*>(smem + L::oP);
  float* sG = reinterpret_cast<float*>(smem + L::oG);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sGam = reinterpret_cast<float*>(smem + L::oGam);
  float* sGamC = reinterpret_cast<float*>(smem + L::oGamC);
  float* sGs = reinterpret_cast<float*>(smem + L::oGs);
  int* sFlag = reinterpret_cast<int*>(smem + L::oFlag);
  CT* sK = reinterpret_cast<CT*>(smem + L::oK);    // channel: K-side factors
  CT* sEb = reinterpret_cast<CT*>(smem + L::oEb);  // channel: Xe (16 rows) then Xq (16 rows)
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  CT* sTb = reinterpret_cast<CT*>(smem + L::oTb);
  float* sFB = reinterpret_cast<float*>(smem + L::oFB);
  float* sScan = reinterpret_cast<float*>(smem + L::oR1);
  CT* sY = reinterpret_cast<CT*>(smem + L::oY);
  CT* sST = reinterpret_cast<CT*>(smem + L::oST);
  CT* sWT = reinterpret_cast<CT*>(smem + L::oWT);

  // views of A: row-major, and its transpose with k contiguous
  const View<CT> vArm = view(sArm, SC, 1);
  View<CT> vAT;  // vAT(n, k) = A[k][n]
  if constexpr (L::CM) vAT = view(sAcm, SC, 1); else vAT = view(sArm, 1, SC);

  // A and A_qk are stored whole; their strictly-upper 16x16 blocks stay zero
  // for the whole kernel (nothing writes them), so triangular products can
  // run over the full 64-wide k range.
  for (int e = tid; e < CH * SC; e += NTHR) {
    sArm[e] = (CT)0.f;
    sAqk[e] = (CT)0.f;
    if constexpr (L::CM) sAcm[e] = (CT)0.f;
  }

  // ---- state slice in accumulators: rows c, columns v -------------------
  f32x4 Sacc[MC][NV];
#pragma unroll
  for (int mt = 0; mt < MC; ++mt)
#pragma unroll
    for (int nt = 0; nt < NV; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = (wave * MC + mt) * 16 + ((lane >> 4) << 2) + r;
        const int v = vbase + nt * 16 + (lane & 15);
        Sacc[mt][nt][r] = p.state_in ? p.state_in[((size_t)bh * DK + c) * DV + v] : 0.f;
      }

  // ---- per-thread prep layout ---------------------------------------------
  const int cg = tid % CG, tg = tid / CG;
  const int c0 = cg * 8, tq0 = tg * TPT;       // 8 channels x TPT tokens
  const int myI = tq0 >> 4;                    // 16-token block of my tokens
  const int vgi = tid % VG, vt = tid / VG;
  const int vv0 = vgi * 8, vtq0 = vt * VPT;    // 8 value columns x VPT tokens (vtq0 may pass 63: idle)
  const bool vact = vtq0 < CH;

  struct Raw {
    V8<IO> k[TPT], q[TPT];
    V8<float> g[TPT], bg[TPT];
    float beta[TPT];
    float gt[TPT];  // scalar log-decay of my tokens
    float gs, bs;  // lane-indexed scalar log-decay and beta (token = lane)
    V8<IO> v[VPT];
    V8<float> w[VPT];
    float vb[VPT];
  };

  // Loads are unconditional, at token indices clamped to T - 1, so that none
  // of them waits; rows past the end are zeroed where they are consumed.
  // With no decay the scalar log-decay is read from a stand-in address (any
  // readable buffer of >= B*T*H floats) and discarded.
  const float* gsrc = has_decay ? g_seq : reinterpret_cast<const float*>(p.q) + seq0;
  auto load_raw = [&](int n, Raw& R) {
    const int t0 = n * CH;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int to = min(t0 + tq0 + u, T - 1) * H;
      R.k[u] = ld8(kg + to * DK + c0);
      R.q[u] = ld8(qg + to * DK + c0);
      if constexpr (CHAN) R.g[u] = ld8(g_seq + to * DK + c0);
      else R.gt[u] = gsrc[to];
      if constexpr (erase_ch) R.bg[u] = ld8(b_seq + to * DK + c0);
      if constexpr (need_beta) R.beta[u] = beta_seq[to];
    }
    {
      const int to = min(t0 + lane, T - 1) * H;
      if constexpr (!CHAN) R.gs = gsrc[to];
      if constexpr (need_beta) R.bs = beta_seq[to];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int to = min(t0 + vtq0 + u, T - 1) * H;
      R.v[u] = ld8(vg_ + to * DV + vv0);
      if constexpr (write_ch) R.w[u] = ld8(w_seq + to * DV + vv0);
      else R.vb[u] = beta_seq[to];
    }
  };

  Raw R;
  if (nchunks > 0) load_raw(0, R);

  // Output tiles of the previous chunk, stored one chunk late: vector memory
  // stores share the load counter, so storing right before the prefetch
  // would make the next chunk's wait for its inputs also wait for them.
  f32x4 pendO[NV];
  int pend_t0 = -1;
  auto store_out = [&](int ct0) {
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int I = rt_I<NV>(t, wave), nt = rt_N<NV>(t, wave);
      const int tt = ct0 + 16 * I + (lane & 15);
      if (tt < T) gst4(og + tt * H * DV + 16 * nt + ((lane >> 4) << 2), pendO[t]);
    }
  };

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * CH;

    // =================== prep ==============================================
    float expGC = 1.f;                 // gamma_C (scalar decay)
    float kr[TPT][8];                  // channel: k * exp(G_s - G)   (K-side, own block)
    float ef[TPT][8], qf[TPT][8];      // channel: e * exp(G - G_s), q * exp(G - G_s)
    float gsI[8];                      // channel: G at the start of my block
    if constexpr (!CHAN) {
      // chunk-local inclusive scan of the scalar log-decay, one token per lane
      const float G = wave_incl_scan((has_decay && t0 + lane < T) ? R.gs : 0.f);
      const float GC = lane_value(G, 63);
      expGC = fexp(GC);
      if (wave == 0) {
        sG[lane] = G;
        sGam[lane] = fexp(G);
        sBeta[lane] = need_beta ? R.bs : 0.f;
      }
      // my tokens' cumulative decay: the scan value before my first token,
      // plus my own tokens' log-decays
      float Gt[TPT];
      {
        float run = __shfl(G, (tq0 + 63) & 63);
        if (tq0 == 0) run = 0.f;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          run += (has_decay && t0 + tq0 + u < T) ? R.gt[u] : 0.f;
          Gt[u] = run;
        }
      }
      const bool eb_is_k = !erase_ch && !qmix;
      float ebar[TPT][8], kt[TPT][8];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = tq0 + u;
        const float gam_t = fexp(Gt[u]), tail_t = fexp(GC - Gt[u]);
        const bool ok = t0 + t < T;
        float kf[8], qv[8], eb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          kf[i] = ok ? R.k[u][i] : 0.f;
          qv[i] = ok ? R.q[u][i] : 0.f;
          if constexpr (erase_ch) eb[i] = R.bg[u][i] * kf[i];
          else eb[i] = qmix ? kf[i] + lam * qv[i] : kf[i];
        }
        st8(sK + t * SK + c0, kf);
        st8(sQ + t * SK + c0, qv);
        if (!eb_is_k) st8(sEb + t * SK + c0, eb);
        float es = gam_t;
        if constexpr (!erase_ch) es *= R.beta[u];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ebar[u][i] = es * eb[i];
          kt[u][i] = tail_t * kf[i];
        }
      }
      // transposed writes: my TPT tokens are contiguous in each row c
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a[TPT], c[TPT];
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          a[u] = ebar[u][i];
          c[u] = kt[u][i];
        }
        stn<TPT>(sEbT + (c0 + i) * SC + tq0, a);
        stn<TPT>(sKtT + (c0 + i) * SC + tq0, c);
      }
    } else {
      // chunk-local inclusive cumsum per key channel: local over my TPT
      // tokens, then a prefix over token groups through LDS
      float Gl[TPT][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          s += (t0 + tq0 + u < T) ? R.g[u][i] : 0.f;
          Gl[u][i] = s;
        }
      }
      if (tid == 0) *sFlag = 0;
      st8(sScan + tg * DK + c0, Gl[TPT - 1]);
      __syncthreads();
      float pre[8], tot[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pre[i] = tot[i] = 0.f;
      for (int t2 = 0; t2 < TG; ++t2) {
        const V8<float> s = ld8(sScan + t2 * DK + c0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          tot[i] += s[i];
          if (t2 < tg) pre[i] += s[i];
        }
      }
      float G[TPT][8];
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) G[u][i] = pre[i] + Gl[u][i];
      if ((tq0 & 15) == 0) st8(sGs + myI * DK + c0, G[0]);
      if (tg == 0) {
        float gc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gc[i] = fexp(tot[i]);
        st8(sGamC + c0, gc);
      }
      __syncthreads();
      {
        const V8<float> s = ld8(sGs + myI * DK + c0);
#pragma unroll
        for (int i = 0; i < 8; ++i) gsI[i] = s[i];
      }
      if (((tq0 + TPT) & 15) == 0) {
        // owner of the block's last token: widest log-decay window
        float wmax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) wmax = fmaxf(wmax, gsI[i] - G[TPT - 1][i]);
        if (!(wmax <= WINDOW_LIMIT)) *sFlag = 1;
      }
      float egs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) egs[i] = fexp(gsI[i]);
      float ebar[TPT][8], kt[TPT][8];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = tq0 + u;
        const bool ok = t0 + t < T;
        float qg2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float kv = ok ? R.k[u][i] : 0.f, qv = ok ? R.q[u][i] : 0.f;
          float e;
          if constexpr (erase_ch) e = R.bg[u][i] * kv;
          else e = R.beta[u] * (qmix ? kv + lam * qv : kv);
          const float f = fexp(G[u][i] - gsI[i]);    // <= 1
          const float rf = fexp(gsI[i] - G[u][i]);   // >= 1, <= exp(window)
          const float tl = fexp(tot[i] - G[u][i]);   // gamma_C / gamma_t <= 1
          const float gm = f * egs[i];                // gamma_t
          ebar[u][i] = gm * e;
          kt[u][i] = tl * kv;
          qg2[i] = gm * qv;
          kr[u][i] = rf * kv;
          ef[u][i] = f * e;
          qf[u][i] = f * qv;
        }
        st8(sQ + t * SK + c0, qg2);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a[TPT], c[TPT];
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          a[u] = ebar[u][i];
          c[u] = kt[u][i];
        }
        stn<TPT>(sEbT + (c0 + i) * SC + tq0, a);
        stn<TPT>(sKtT + (c0 + i) * SC + tq0, c);
      }
    }
    // value side: Z^T (my VPT tokens are contiguous in each row v)
    if (vact) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float z[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          float gate;
          if constexpr (write_ch) gate = R.w[u][i];
          else gate = R.vb[u];
          z[u] = (t0 + vtq0 + u < T) ? gate * R.v[u][i] : 0.f;
        }
        stn<VPT>(sZT + (vv0 + i) * SC + vtq0, z);
      }
    }
    __syncthreads();

    if (pend_t0 >= 0) store_out(pend_t0);
    // prefetch the next chunk while this one is processed
    if (n + 1 < nchunks) load_raw(n + 1, R);

    // =================== gram: T and A_qk ===================================
    if constexpr (!CHAN) {
      const bool eb_is_k = !erase_ch && !qmix;
      const View<CT> vK = view(sK, SK, 1);
      const View<CT> vE = view(eb_is_k ? sK : sEb, SK, 1);
      const View<CT> vQ = view(sQ, SK, 1);
      // 10 lower block pairs (I >= J) x {T, A_qk}: wave w takes tasks
      // w, w + 4, ..., i.e. kind = w & 1 and pairs (w >> 1) + 2 m
      const int kind = wave & 1;
      const View<CT> vB = kind ? vQ : vE;
      const float* gsrc_lds = sG;
      f32x4 acc[5];
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const int pr = (wave >> 1) + 2 * m;
        acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[m] = tmm<DK>(acc[m], vK, 16 * pair_J(pr), 0, vB, 16 * pair_I(pr), 0, lane);
      }
      // decay, gate and mask; all LDS reads first, then the stores
      float Gi[5], gi[5];
      f32x4 Gj[5];
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const int pr = (wave >> 1) + 2 * m;
        const int i = 16 * pair_I(pr) + (lane & 15);
        Gi[m] = gsrc_lds[i];
        gi[m] = sBeta[i];
        Gj[m] = *reinterpret_cast<const f32x4*>(gsrc_lds + 16 * pair_J(pr) + ((lane >> 4) << 2));
      }
      CT* dst = kind ? sAqk : sTb;
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const int pr = (wave >> 1) + 2 * m;
        const int I = pair_I(pr), J = pair_J(pr);
        const int i = 16 * I + (lane & 15);
        const int j0 = 16 * J + ((lane >> 4) << 2);
        const float gate = (kind || erase_ch) ? 1.f : gi[m];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = gate * acc[m][r] * fexp(Gi[m] - Gj[m][r]);
          acc[m][r] = (j0 + r < i + kind) ? x : 0.f;  // T: j < i; A_qk: j <= i
        }
        tst_vec(view(dst, 1, SC), 16 * J, 16 * I, acc[m], lane);
      }
      // the fp32 diagonal blocks of T for the substitution (waves 0 and 2
      // hold T tiles; their diagonal pairs are m = 0, 2 (wave 0) and 1, 4 (wave 2))
      if (!kind) {
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const int pr = (wave >> 1) + 2 * m;
          const int I = pair_I(pr), J = pair_J(pr);
          if (I == J) tst_sca(view(sTd + I * 16 * TDS, TDS, 1), 0, 0, acc[m], lane);
        }
      }
      __syncthreads();
    } else {
      // Bounded factors: row block I uses the reference token s = 16 I.
      //   x_i * exp(G_i - G_s)   (<= 1, i in block I)
      //   k_j * exp(G_s - G_j)   (<= 1 for j < s; <= exp(window) for j in block I)
      // Their product over channels is exactly the entry.  Upper-triangle
      // entries of the diagonal tiles may be huge; they are masked.
      CT* sXe = sEb;
      CT* sXq = sEb + 16 * SK;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if (myI <= I) {
          float fk[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            fk[i] = (myI == I) ? 1.f : fexp(sGs[I * DK + c0 + i] - gsI[i]);
#pragma unroll
          for (int u = 0; u < TPT; ++u) {
            float kh[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) kh[i] = kr[u][i] * fk[i];
            st8(sK + (tq0 + u) * SK + c0, kh);
          }
          if (myI == I) {
#pragma unroll
            for (int u = 0; u < TPT; ++u) {
              st8(sXe + (tq0 - 16 * I + u) * SK + c0, ef[u]);
              st8(sXq + (tq0 - 16 * I + u) * SK + c0, qf[u]);
            }
          }
        }
        __syncthreads();
        f32x4 acc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int task = wave + 4 * m;
          acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (task < 2 * (I + 1))
            acc[m] = tmm<DK>(acc[m], view(sK, SK, 1), 16 * (task >> 1), 0, view((task & 1) ? sXq : sXe, SK, 1), 0,
                             0, lane);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int task = wave + 4 * m;
          if (task < 2 * (I + 1)) {
            const int J = task >> 1, kind = task & 1;
            const int i = 16 * I + (lane & 15);
            f32x4 val;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * J + ((lane >> 4) << 2) + r;
              val[r] = (kind ? (j <= i) : (j < i)) ? acc[m][r] : 0.f;
            }
            if (kind) {
              tst_vec(view(sAqk, 1, SC), 16 * J, 16 * I, val, lane);
            } else {
              tst_vec(view(sTb, 1, SC), 16 * J, 16 * I, val, lane);
              if (I == J) tst_sca(view(sTd + I * 16 * TDS, TDS, 1), 0, 0, val, lane);
            }
          }
        }
        __syncthreads();
      }

      // Fallback for chunks where some 16-token window decays by more than
      // WINDOW_LIMIT in some channel: every lower entry is recomputed as
      // sum_c x_i[c] k_j[c] exp(G_i[c] - G_j[c]) with the exponent <= 0,
      // from the chunk's inputs re-read from global memory.
      if (*sFlag) {
        constexpr int FBC = L::FBC, FBS = L::FBS;
        constexpr int NPAIR = CH * (CH + 1) / 2;       // 2080 lower pairs (with diagonal)
        constexpr int PPT = (NPAIR + NTHR - 1) / NTHR; // 9
        float accT[PPT], accA[PPT];
#pragma unroll
        for (int m = 0; m < PPT; ++m) accT[m] = accA[m] = 0.f;
        float* fG = sFB;
        float* fE = sFB + CH * FBS;
        float* fK = sFB + 2 * CH * FBS;
        float* fQ = sFB + 3 * CH * FBS;
        for (int cs = 0; cs < DK; cs += FBC) {
          // stage 64 tokens x FBC channels (each thread: 2 elements)
          for (int e = tid; e < CH * FBC; e += NTHR) {
            const int t = e / FBC, ch = e % FBC, c = cs + ch;
            const bool ok = t0 + t < T;
            const int to = min(t0 + t, T - 1) * H;
            const float kv = ok ? (float)kg[to * DK + c] : 0.f;
            const float qv = ok ? (float)qg[to * DK + c] : 0.f;
            const float gv = ok ? g_seq[to * DK + c] : 0.f;
            float ev;
            if constexpr (erase_ch) ev = (ok ? b_seq[to * DK + c] : 0.f) * kv;
            else ev = (ok ? beta_seq[to] : 0.f) * (qmix ? kv + lam * qv : kv);
            fG[t * FBS + ch] = gv;
            fE[t * FBS + ch] = ev;
            fK[t * FBS + ch] = kv;
            fQ[t * FBS + ch] = qv;
          }
          __syncthreads();
          if (tid < FBC) {
            float s = 0.f;
            for (int t = 0; t < CH; ++t) {
              s += fG[t * FBS + tid];
              fG[t * FBS + tid] = s;
            }
          }
          __syncthreads();
#pragma unroll
          for (int m = 0; m < PPT; ++m) {
            const int pp = tid + m * NTHR;
            if (pp < NPAIR) {
              int i = (int)((sqrtf(8.f * pp + 1.f) - 1.f) * 0.5f);
              while ((i + 1) * (i + 2) / 2 <= pp) ++i;
              while (i * (i + 1) / 2 > pp) --i;
              const int j = pp - i * (i + 1) / 2;
              float st = 0.f, sa = 0.f;
#pragma unroll
              for (int ch = 0; ch < FBC; ++ch) {
                const float x = fexp(fG[i * FBS + ch] - fG[j * FBS + ch]) * fK[j * FBS + ch];
                st += fE[i * FBS + ch] * x;
                sa += fQ[i * FBS + ch] * x;
              }
              accT[m] += st;
              accA[m] += sa;
            }
          }
          __syncthreads();
        }
#pragma unroll
        for (int m = 0; m < PPT; ++m) {
          const int pp = tid + m * NTHR;
          if (pp < NPAIR) {
            int i = (int)((sqrtf(8.f * pp + 1.f) - 1.f) * 0.5f);
            while ((i + 1) * (i + 2) / 2 <= pp) ++i;
            while (i * (i + 1) / 2 > pp) --i;
            const int j = pp - i * (i + 1) / 2;
            const float tv = (j < i) ? accT[m] : 0.f;
            sTb[i * SC + j] = (CT)tv;
            if ((i >> 4) == (j >> 4)) sTd[(i >> 4) * 16 * TDS + (j & 15) * TDS + (i & 15)] = tv;
            sAqk[i * SC + j] = (CT)accA[m];
          }
        }
        __syncthreads();
      }
    }

    // =================== solve: A = (I + T)^{-1} ============================
    // level 0: wave w inverts diagonal block w by column-sweep substitution;
    // lane c (< 16) owns column c of A_ww.  sTd holds each block as T^T
    // (row j of sTd = column j of T), read with uniform (broadcast) loads.
    {
      const float* Td = sTd + wave * 16 * TDS;
      const int c = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
      // column j needs rows j+1..15: the aligned float4 groups from (j+1)/4
      f32x4 col[15][4];
#pragma unroll
      for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int q4 = (j + 1) / 4; q4 < 4; ++q4) col[j][q4] = *reinterpret_cast<const f32x4*>(Td + j * TDS + 4 * q4);
#pragma unroll
      for (int j = 0; j < 15; ++j)
#pragma unroll
        for (int i = j + 1; i < 16; ++i) x[i] -= col[j][i >> 2][i & 3] * x[j];
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sArm[(16 * wave + i) * SC + 16 * wave + c] = (CT)x[i];
        if constexpr (L::CM) {
          float lo[8], hi[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            lo[i] = x[i];
            hi[i] = x[i + 8];
          }
          st8(sAcm + (16 * wave + c) * SC + 16 * wave, lo);
          st8(sAcm + (16 * wave + c) * SC + 16 * wave + 8, hi);
        }
      }
    }
    __syncthreads();
    // level 1: A_10 (wave 0) and A_32 (wave 1): A_IJ = -A_II (T_IJ A_JJ)
    if (wave < 2) {
      const int I = 2 * wave + 1, J = 2 * wave;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tmm_exact<16>(acc, view(sTb, SC, 1), 16 * I, 16 * J, vAT, 16 * J, 16 * J, lane);
      tst_vec(view(sP + wave * 16 * SP, 1, SP), 0, 0, acc, lane);  // P^T row-major
    }
    __syncthreads();
    if (wave < 2) {
      const int I = 2 * wave + 1, J = 2 * wave;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tmm_exact<16>(acc, vArm, 16 * I, 16 * I, view(sP + wave * 16 * SP, SP, 1), 0, 0, lane);
      acc = -acc;
      tst_sca(view(sArm, SC, 1), 16 * I, 16 * J, acc, lane);
      if constexpr (L::CM) tst_vec(view(sAcm, 1, SC), 16 * I, 16 * J, acc, lane);
    }
    __syncthreads();
    // level 2: rows 32..63 x columns 0..31:
    //   P_IJ = T[I, 0:32] A[0:32, J]   (A's upper block (0,1) is zero)
    //   A_IJ = -A[I, 32:64] P[32:64, J]
    {
      const int I = 2 + (wave >> 1), J = wave & 1;
      CT* P2 = sP + J * 16 * SP2;  // P tiles (2,J) and (3,J), stacked along k
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tmm<32>(acc, view(sTb, SC, 1), 16 * I, 0, vAT, 16 * J, 0, lane);
      tst_vec(view(P2 + (I - 2) * 16, 1, SP2), 0, 0, acc, lane);
    }
    __syncthreads();
    {
      const int I = 2 + (wave >> 1), J = wave & 1;
      CT* P2 = sP + J * 16 * SP2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = tmm<32>(acc, vArm, 16 * I, 32, view(P2, SP2, 1), 0, 0, lane);
      acc = -acc;
      tst_sca(view(sArm, SC, 1), 16 * I, 16 * J, acc, lane);
      if constexpr (L::CM) tst_vec(view(sAcm, 1, SC), 16 * I, 16 * J, acc, lane);
    }
    __syncthreads();

    // =================== wy: Y^T = E_bar^T A^T, U = A Z; S^T to LDS ==========
    f32x4 accY[DK / 64][4];
#pragma unroll
    for (int cbi = 0; cbi < DK / 64; ++cbi)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        accY[cbi][I] = f32x4{0.f, 0.f, 0.f, 0.f};
        accY[cbi][I] = tmm<CH>(accY[cbi][I], view(sEbT, SC, 1), 16 * (wave + 4 * cbi), 0, vArm, 16 * I, 0, lane);
      }
    f32x4 accW[NV];
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      accW[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      accW[t] = tmm<CH>(accW[t], vArm, 16 * rt_I<NV>(t, wave), 0, view(sZT, SC, 1), 16 * rt_N<NV>(t, wave), 0,
                        lane);
    }
#pragma unroll
    for (int cbi = 0; cbi < DK / 64; ++cbi)
#pragma unroll
      for (int I = 0; I < 4; ++I)
        tst_vec(view(sY, 1, SK), 16 * (wave + 4 * cbi), 16 * I, -accY[cbi][I], lane);  // -Y, row-major [i][c]
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
      for (int nt = 0; nt < NV; ++nt)
        tst_vec(view(sST, 1, SK), (wave * MC + mt) * 16, nt * 16, Sacc[mt][nt], lane);
    __syncthreads();

    // =================== state: W = U - Y S, O^T = S^T Q^T + W^T A_qk^T ======
    f32x4 accO[NV];
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int I = rt_I<NV>(t, wave), nt = rt_N<NV>(t, wave);
      accW[t] = tmm<DK>(accW[t], view(sY, SK, 1), 16 * I, 0, view(sST, SK, 1), 16 * nt, 0, lane);
      accO[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      accO[t] = tmm<DK>(accO[t], view(sST, SK, 1), 16 * nt, 0, view(sQ, SK, 1), 16 * I, 0, lane);
    }
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int I = rt_I<NV>(t, wave), nt = rt_N<NV>(t, wave);
      tst_vec(view(sWT, 1, SC), 16 * I, 16 * nt, accW[t], lane);
      if constexpr (!CHAN) accO[t] *= sGam[16 * I + (lane & 15)];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int I = rt_I<NV>(t, wave), nt = rt_N<NV>(t, wave);
      pendO[t] = tmm<CH>(accO[t], view(sWT, SC, 1), 16 * nt, 0, view(sAqk, SC, 1), 16 * I, 0, lane);
    }
    pend_t0 = t0;
#pragma unroll
    for (int mt = 0; mt < MC; ++mt) {
      const int cb = wave * MC + mt;
      f32x4 gc;
      if constexpr (CHAN) gc = *reinterpret_cast<const f32x4*>(sGamC + cb * 16 + ((lane >> 4) << 2));
      else gc = f32x4{expGC, expGC, expGC, expGC};
#pragma unroll
      for (int nt = 0; nt < NV; ++nt) {
        Sacc[mt][nt] *= gc;
        Sacc[mt][nt] = tmm<CH>(Sacc[mt][nt], view(sKtT, SC, 1), cb * 16, 0, view(sWT, SC, 1), 16 * nt, 0, lane);
      }
    }
    __syncthreads();
  }

  if (pend_t0 >= 0) store_out(pend_t0);
  if (p.state_out) {
#pragma unroll
    for (int mt = 0; mt < MC; ++mt)
#pragma unroll
      for (int nt = 0; nt < NV; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = (wave * MC + mt) * 16 + ((lane >> 4) << 2) + r;
          const int v = vbase + nt * 16 + (lane & 15);
          p.state_out[((size_t)bh * DK + c) * DV + v] = Sacc[mt][nt][r];
        }
  }
}

template <class CT, int DK, int DVS, bool CHAN>
constexpr int chunk_lds_bytes() {
  return Lay<CT, DK, DVS, CHAN>::TOTAL;
}

}  // namespace gdr
