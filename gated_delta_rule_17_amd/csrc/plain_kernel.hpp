// Plain fp32 chunk kernel: the chunk WY form with absorbed decay of "Gated
// DeltaNet-2: Decoupling Erase and Write in Linear Attention" (key design 2)
// evaluated entirely in fp32 on the vector ALUs, for every variant and gate
// kind the library accepts.
//
// It serves the cases the MFMA kernels do not cover:
//  - fp32 I/O at dk = 128 (the fp32 operand tiles of the MFMA kernels do not
//    fit the 160 KB of LDS at that width);
//  - a time-varying Q-Delta coefficient lambda_t ("Q-Delta: Beyond Key-Value
//    Associative State Evolution", key design 2 writes lambda_t in [0, 1]);
//  - a write strength per value channel ("Chapter 11 Gated DeltaNet", 11.3:
//    the module gates the prediction error of each value channel with its own
//    beta, so each state column follows its own scalar-beta delta rule).
//
// Per chunk of C = 64 tokens, with G the chunk-local inclusive cumsum of the
// log-decay (per key channel; a scalar decay is broadcast over the channels)
// and S the fp32 state slice entering the chunk:
//   T[i][j]   = sum_c e_i[c] k_j[c] exp(G_i[c] - G_j[c])      j <  i
//   Aqk[i][j] = sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])      j <= i
//   ES[i][v]  = sum_c e_i[c] exp(G_i[c]) S[c][v]               (E_bar S)
//   QS[i][v]  = sum_c q_i[c] exp(G_i[c]) S[c][v]               (Q_gamma S)
//   W         solves (I + M (.) T) W = Z - M (.) ES by forward substitution
//   O         = QS + Aqk W
//   S        <- Diag(exp(G_C)) S + K_tail^T W,  K_tail[j][c] = k_j[c] exp(G_C[c] - G_j[c])
// Every exponent is <= 0, so no factor leaves the fp32 range (the page's
// gamma^{-1} is never formed).  M is 1, except under the per-value-channel
// beta, where e = k and M[i][v] = beta_i[v] scales row i of the system of
// column v (the forward substitution then runs per column, which is what
// "needs dv solves per chunk" costs: one substitution per column).  W is
// the page's U - Y S = A (Z - E_bar S), solved for directly.
//
// One workgroup (4 waves) owns one (batch, head) and a slice of DVS = 16
// value columns; chunks are walked in order, the slice of the state stays in
// LDS.  q, k, e, G rows of the chunk are staged in LDS as fp32.
//
// Record mode (REC) is the first pass of the backward: instead of o it
// writes, per chunk, what the reverse passes read back (see bwd_kernel.hpp):
// the entering state and W (each slice its columns), and, from slice 0, T,
// A_qk, E_bar, Q_gamma, K_tail and gamma_C.
#pragma once

#include "bwd_params.hpp"
#include "chunk_kernel.hpp"

namespace gdr {


template <int DK, int DVS>
struct PlainLay {
  static constexpr int DKP = DK + 1;   // row stride (floats) of [64][DK] arrays
  static constexpr int DVP = DVS + 1;  // row stride of [rows][DVS] arrays
  static constexpr int TP = CH + 1;    // row stride of [64][64] arrays
  // float offsets
  static constexpr int oK = 0;                 // [64][DKP] k
  static constexpr int oX = oK + CH * DKP;     // [64][DKP] erase directions e
  static constexpr int oQ = oX + CH * DKP;     // [64][DKP] q
  static constexpr int oG = oQ + CH * DKP;     // [64][DKP] chunk-local cumsum of the log-decay
  static constexpr int oS = oG + CH * DKP;     // [DK][DVP] state slice
  static constexpr int oZ = oS + DK * DVP;     // [64][DVP] written values z
  static constexpr int oM = oZ + CH * DVP;     // [64][DVP] erase multiplier M
  static constexpr int oW = oM + CH * DVP;     // [64][DVP] W
  static constexpr int END = oW + CH * DVP;
  // after the Gram: T, A_qk, E_bar S, Q_gamma S, in the space of X and Q
  // where they fit (dk = 128), else after the other arrays
  static constexpr int POST = 2 * CH * TP + 2 * CH * DVP;
  static constexpr bool OVERLAY = POST <= 2 * CH * DKP;
  static constexpr int oT = OVERLAY ? oX : END;  // [64][TP]  T (strictly lower)
  static constexpr int oAqk = oT + CH * TP;      // [64][TP]  A_qk (lower, diagonal included)
  static constexpr int oES = oAqk + CH * TP;     // [64][DVP] E_bar S
  static constexpr int oQS = oES + CH * DVP;     // [64][DVP] Q_gamma S
  static constexpr int TOTAL = OVERLAY ? END : END + POST;
  static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget exceeded");
};

template <int DK, int DVS>
constexpr int plain_lds_bytes() {
  return PlainLay<DK, DVS>::TOTAL * 4;
}

__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const bf16* p) { return (float)*p; }
__device__ __forceinline__ f32x4 ldf4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ldf4(const bf16* p) {
  return __builtin_convertvector(*reinterpret_cast<const bf16x4*>(p), f32x4);
}

// Loads kept in the I/O type until their use: a record loaded a chunk ahead
// and widened where it is consumed, so that no conversion right after the
// load makes the wave wait for it there.
template <class IO>
struct Raw;
template <>
struct Raw<float> {
  typedef f32x4 v4;
};
template <>
struct Raw<bf16> {
  typedef bf16x4 v4;
};
template <class IO>
__device__ __forceinline__ typename Raw<IO>::v4 ldraw4(const IO* p) {
  return *reinterpret_cast<const typename Raw<IO>::v4*>(p);
}
__device__ __forceinline__ f32x4 widen(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 widen(bf16x4 x) { return __builtin_convertvector(x, f32x4); }

// sum over the 16 lanes of each 16-lane group
__device__ __forceinline__ float sum16(float s) {
  s += __shfl_xor(s, 1, 16);
  s += __shfl_xor(s, 2, 16);
  s += __shfl_xor(s, 4, 16);
  s += __shfl_xor(s, 8, 16);
  return s;
}

template <class IO, int DK, int DVS, bool REC = false>
__global__ __launch_bounds__(NTHR) void plain_fwd_kernel(ChunkParams p, BwdWs ws) {
  using L = PlainLay<DK, DVS>;
  constexpr int DKP = L::DKP, DVP = L::DVP, TP = L::TP;
  static_assert(DVS == 16, "the substitution maps 16 columns x 16 lanes onto the workgroup");
  __shared__ __attribute__((aligned(16))) float lds[L::TOTAL];
  float* sK = lds + L::oK;
  float* sX = lds + L::oX;
  float* sQ = lds + L::oQ;
  float* sG = lds + L::oG;
  float* sS = lds + L::oS;
  float* sZ = lds + L::oZ;
  float* sM = lds + L::oM;
  float* sW = lds + L::oW;
  float* sT = lds + L::oT;
  float* sAqk = lds + L::oAqk;
  float* sES = lds + L::oES;
  float* sQS = lds + L::oQS;

  const int tid = threadIdx.x;
  const int NS = p.nslices;
  const int bh = blockIdx.x / NS, slice = blockIdx.x - bh * NS;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H, DV = p.DV;
  const int vbase = slice * DVS;
  const int nchunks = (T + CH - 1) / CH;
  const int decay = p.decay, erase = p.erase, write = p.write, qmix = p.qmix;

  // token index of (bb, t = 0, hh); per-token tensors are [B, T, H, .]
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* qg = reinterpret_cast<const IO*>(p.q);
  const IO* kg = reinterpret_cast<const IO*>(p.k);
  const IO* vg = reinterpret_cast<const IO*>(p.v);
  IO* og = reinterpret_cast<IO*>(p.o);

  // state slice in
  for (int e = tid; e < DK * DVS; e += NTHR) {
    const int c = e / DVS, v = e - c * DVS;
    sS[c * DVP + v] = p.state_in ? p.state_in[((size_t)bh * DK + c) * DV + vbase + v] : 0.f;
  }

  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * CH;
    const size_t ch = (size_t)bh * nchunks + n;
    if constexpr (REC) {
      for (int e = tid; e < DK * DVS; e += NTHR) {
        const int c = e / DVS, v = e - c * DVS;
        ws.S[(ch * DK + c) * DV + vbase + v] = sS[c * DVP + v];
      }
    }
    // ---- rows of the chunk: k, q, e and the log-decay (zero past T).  Four
    // channels per load; every load of the chunk is issued first, at a token
    // index clamped to T - 1, and masked afterwards.
    {
      constexpr int QPR = DK / 4, NQ = CH * QPR / NTHR;
      f32x4 rk[NQ], rq[NQ], rg[NQ], rb[NQ];
      float rgs[NQ], rbe[NQ], rl[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int e = tid + NTHR * u, r = e / QPR, c4 = (e - r * QPR) * 4;
        const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
        rk[u] = ldf4(kg + tok * DK + c4);
        rq[u] = ldf4(qg + tok * DK + c4);
        if (decay == 2) rg[u] = ldf4(p.g + tok * DK + c4);
        rgs[u] = decay == 1 ? p.g[tok] : 0.f;
        if (erase == 1) rb[u] = ldf4(p.b + tok * DK + c4);
        rbe[u] = erase == 0 ? p.beta[tok] : 0.f;
        rl[u] = qmix == 2 ? p.lam[tok] : (qmix ? p.lam[hh] : 0.f);
      }
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int e = tid + NTHR * u, r = e / QPR, c4 = (e - r * QPR) * 4;
        const bool ok = t0 + r < T;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float kv = ok ? rk[u][i] : 0.f, qv = ok ? rq[u][i] : 0.f;
          float ev;
          if (erase == 1) ev = rb[u][i] * kv;
          else if (erase == 2) ev = kv;  // per-value-channel beta: the strength sits in M
          else ev = rbe[u] * __builtin_fmaf(rl[u], qv, kv);
          sK[r * DKP + c4 + i] = kv;
          sQ[r * DKP + c4 + i] = qv;
          sX[r * DKP + c4 + i] = ok ? ev : 0.f;
          sG[r * DKP + c4 + i] = !ok ? 0.f : (decay == 2 ? rg[u][i] : rgs[u]);
        }
      }
    }
    // ---- value side: z and the erase multiplier M -------------------------
    {
      constexpr int NV = CH * DVS / NTHR;
      float rv[NV], rw[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = tid + NTHR * u, r = e / DVS, v = e - r * DVS;
        const size_t tok = seq0 + (size_t)min(t0 + r, T - 1) * H;
        rv[u] = ldf(vg + tok * DV + vbase + v);
        rw[u] = erase == 2 ? p.beta[tok * DV + vbase + v] : (write == 1 ? p.w[tok * DV + vbase + v] : p.beta[tok]);
      }
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = tid + NTHR * u, r = e / DVS, v = e - r * DVS;
        const bool ok = t0 + r < T;
        sZ[r * DVP + v] = ok ? rw[u] * rv[u] : 0.f;
        sM[r * DVP + v] = (ok && erase == 2) ? rw[u] : 1.f;
      }
    }
    __syncthreads();
    // ---- chunk-local inclusive cumsum of the log-decay, one channel per thread
    if (tid < DK) {
      float run = 0.f;
      for (int r = 0; r < CH; ++r) {
        run += sG[r * DKP + tid];
        sG[r * DKP + tid] = run;
      }
    }
    __syncthreads();
    if constexpr (REC) {
      if (slice == 0) {
        for (int e = tid; e < CH * DK; e += NTHR) {
          const int r = e / DK, c = e - r * DK;
          const float G = sG[r * DKP + c], GC = sG[(CH - 1) * DKP + c], gam = fexp(G);
          ws.Eb[(ch * CH + r) * DK + c] = sX[r * DKP + c] * gam;
          ws.Qg[(ch * CH + r) * DK + c] = sQ[r * DKP + c] * gam;
          ws.Kt[(ch * CH + r) * DK + c] = sK[r * DKP + c] * fexp(GC - G);
          if (r == 0) ws.gC[ch * DK + c] = fexp(GC);
        }
      }
    }

    // ---- Gram: T and A_qk, 4 x 4 (i, j) blocks per thread ----------------
    float accT[4][4], accA[4][4];
    const int ib = tid >> 4, jb = tid & 15;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) accT[a][b] = accA[a][b] = 0.f;
    if (jb <= ib) {
      for (int c = 0; c < DK; ++c) {
        float xi[4], qi[4], gi[4], kj[4], gj[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int i = 4 * ib + a, j = 4 * jb + a;
          xi[a] = sX[i * DKP + c];
          qi[a] = sQ[i * DKP + c];
          gi[a] = sG[i * DKP + c];
          kj[a] = sK[j * DKP + c];
          gj[a] = sG[j * DKP + c];
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
    // ---- E_bar S and Q_gamma S: row i, 4 columns per thread ---------------
    float es[4] = {0.f, 0.f, 0.f, 0.f}, qs[4] = {0.f, 0.f, 0.f, 0.f};
    const int ri = tid >> 2, vq = (tid & 3) * 4;
    for (int c = 0; c < DK; ++c) {
      const float gam = fexp(sG[ri * DKP + c]);
      const float xe = sX[ri * DKP + c] * gam, xq = sQ[ri * DKP + c] * gam;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float s = sS[c * DVP + vq + u];
        es[u] = __builtin_fmaf(xe, s, es[u]);
        qs[u] = __builtin_fmaf(xq, s, qs[u]);
      }
    }
    __syncthreads();  // every read of X and Q is done: their space is reused
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = 4 * ib + a, j = 4 * jb + b;
        sT[i * TP + j] = j < i ? accT[a][b] : 0.f;
        sAqk[i * TP + j] = j <= i ? accA[a][b] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sES[ri * DVP + vq + u] = es[u];
      sQS[ri * DVP + vq + u] = qs[u];
    }
    __syncthreads();
    if constexpr (REC) {
      if (slice == 0) {
        for (int e = tid; e < CH * CH; e += NTHR) {
          const int i = e >> 6, j = e & 63;
          ws.T[ch * CH * CH + e] = sT[i * TP + j];
          ws.A[ch * CH * CH + e] = sAqk[i * TP + j];
        }
      }
    }

    // ---- W: forward substitution, column v = tid / 16, lanes split j ------
    {
      const int v = tid >> 4, part = tid & 15;
      float wreg[4] = {0.f, 0.f, 0.f, 0.f};  // W[part + 16 m][v]
      for (int i = 0; i < CH; ++i) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int j = part + 16 * m;
          if (j < i) s = __builtin_fmaf(sT[i * TP + j], wreg[m], s);
        }
        s = sum16(s);
        const float w = sZ[i * DVP + v] - sM[i * DVP + v] * (sES[i * DVP + v] + s);
        if ((i & 15) == part) wreg[i >> 4] = w;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sW[(part + 16 * m) * DVP + v] = wreg[m];
        if constexpr (REC) ws.W[(ch * CH + part + 16 * m) * DV + vbase + v] = wreg[m];
      }
    }
    __syncthreads();

    // ---- O = Q_gamma S + A_qk W -------------------------------------------
    {
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = sQS[ri * DVP + vq + u];
      for (int j = 0; j <= ri; ++j) {
        const float a = sAqk[ri * TP + j];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = __builtin_fmaf(a, sW[j * DVP + vq + u], o[u]);
      }
      const int t = t0 + ri;
      if (!REC && t < T) {
        IO* op = og + (seq0 + (size_t)t * H) * DV + vbase + vq;
#pragma unroll
        for (int u = 0; u < 4; ++u) op[u] = (IO)o[u];
      }
    }
    // ---- S <- Diag(gamma_C) S + K_tail^T W: 8 entries of one row per thread
    {
      const int c = tid >> 1, v0 = (tid & 1) * 8;
      if (c < DK) {
        const float GC = sG[(CH - 1) * DKP + c];
        const float gC = fexp(GC);
        float s[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] = gC * sS[c * DVP + v0 + u];
        for (int j = 0; j < CH; ++j) {
          const float kt = sK[j * DKP + c] * fexp(GC - sG[j * DKP + c]);
#pragma unroll
          for (int u = 0; u < 8; ++u) s[u] = __builtin_fmaf(kt, sW[j * DVP + v0 + u], s[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) sS[c * DVP + v0 + u] = s[u];
      }
    }
    __syncthreads();
  }

  if (p.state_out) {
    for (int e = tid; e < DK * DVS; e += NTHR) {
      const int c = e / DVS, v = e - c * DVS;
      p.state_out[((size_t)bh * DK + c) * DV + vbase + v] = sS[c * DVP + v];
    }
  }
}

}  // namespace gdr
