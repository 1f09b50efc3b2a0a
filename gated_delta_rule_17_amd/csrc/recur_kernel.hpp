// Fused multi-token recurrent kernel and the output epilogue.
//
// Recurrent form: the token loop of the generalized gated delta rule, the
// "fully recurrent" kernel that the Q-Delta page (key design 3) pairs with
// the chunked one, for short sequences (prefill of a few tokens, speculative
// decode, a streaming caller handing its state back in, "Chapter 11 Gated
// DeltaNet" 11.3).  Per token:
//   S_bar = Diag(alpha_t) S;  r = S_bar^T e_t;  S = S_bar + k_t (z_t - m_t (.) r)^T;  o_t = S^T q_t
// with m_t = 1, or the per-value-channel beta of 11.3 (e = k, z = beta (.) v).
//
// One workgroup per (batch, head) with one thread per value column: thread
// v keeps the columns 2 (v / 2) and 2 (v / 2) + 1 of the state in registers
// for the whole call, over half of the key channels (v % 2 picks the half),
// so each broadcast of a key-side value feeds two columns, the contractions
// over the key channels (r and o) are thread-local up to one exchange with
// the neighbouring lane (DPP), and a token needs no barrier.  The per-token
// key-side vectors (alpha, e, k, q) of a block of TB = 8 tokens are staged in
// LDS and read as broadcasts; thread v stages and writes column v.
//
// Output epilogue (11.3: RMSNorm of each head's readout, then the SiLU output
// gate; the Gated DeltaNet-2 page's method flowchart ends with the same step):
//   y = o / sqrt(mean_v(o^2) + eps) * weight (.) silu(gate),  silu(x) = x / (1 + exp(-x))
// fused into the recurrent kernel (the workgroup holds a token's whole
// readout), and as a standalone kernel over rows of o.
#pragma once

#include "common.hpp"

namespace gdr {

struct RecurParams {
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
  const void* gate;  // epilogue: [B,T,H,dv] io dtype, or nullptr (plain readout)
  const float* nw;   // epilogue: RMSNorm weight [dv]
  float eps;
  int B, T, H;
  int decay, erase, write, qmix;
};

__device__ __forceinline__ float ldx(const float* p) { return *p; }
__device__ __forceinline__ float ldx(const bf16* p) { return (float)*p; }

// four consecutive elements as floats
__device__ __forceinline__ f32x4 ld4x(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4x(const bf16* p) {
  return __builtin_convertvector(*reinterpret_cast<const bf16x4*>(p), f32x4);
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + fexp(-x)); }

template <class IO, int DK, int DV>
__global__ __launch_bounds__(DV) void recur_fwd_kernel(RecurParams p) {
  constexpr int TB = 8;         // tokens staged per block
  constexpr int NW = DV / 64;   // waves
  static_assert(DV % 64 == 0 && DK % 4 == 0, "recurrent layout");
  __shared__ __attribute__((aligned(16))) float sA[TB][DK], sE[TB][DK], sK[TB][DK], sQ[TB][DK];
  __shared__ float sP[TB][NW];
  __shared__ float sZ[TB][DV], sM[TB][DV], sGt[TB][DV];  // value side, one column per thread

  const int v = threadIdx.x, wave = v >> 6;
  const int bh = blockIdx.x;
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int T = p.T, H = p.H;
  const int decay = p.decay, erase = p.erase, write = p.write, qmix = p.qmix;
  const size_t seq0 = (size_t)bb * T * H + hh;
  const IO* qg = reinterpret_cast<const IO*>(p.q);
  const IO* kg = reinterpret_cast<const IO*>(p.k);
  const IO* vg = reinterpret_cast<const IO*>(p.v);
  const IO* gateg = reinterpret_cast<const IO*>(p.gate);
  IO* og = reinterpret_cast<IO*>(p.o);
  const bool epi = p.gate != nullptr;
  const float nwv = epi ? p.nw[v] : 0.f;

  // state: columns col0 and col0 + 1, key channels cb .. cb + DK / 2 - 1
  constexpr int DH = DK / 2;
  const int col0 = v & ~1, hf = v & 1, cb = hf * DH;
  float S[2][DH];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int c = 0; c < DH; ++c)
      S[j][c] = p.state_in ? p.state_in[((size_t)bh * DK + cb + c) * DV + col0 + j] : 0.f;
  // the neighbouring lane's partial sum added (DPP quad permutation 1 0 3 2)
  auto pair_sum = [](float x) __attribute__((always_inline)) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, true));
  };

  // staging layout: QPR threads cover a row of DK channels four at a time;
  // the DV / QPR groups of them take every (DV / QPR)-th token of a block
  constexpr int QPR = DK / 4, NG = DV / QPR, TPG = TB / NG;
  static_assert(NG * QPR == DV && TPG * NG == TB, "staging layout");
  const int grp = v / QPR, c4 = (v - grp * QPR) * 4;
  const float* gsrc = decay ? p.g : reinterpret_cast<const float*>(p.v);  // any readable stand-in
  const float* bsrc = (erase == 0 || write == 0) ? p.beta : reinterpret_cast<const float*>(p.v);
  for (int t0 = 0; t0 < T; t0 += TB) {
    const int nt = min(TB, T - t0);
    // ---- key side of the block: alpha, e, k, q (zeros and alpha = 1 past T).
    // Every load is issued first, at a token index clamped to T - 1, and
    // masked afterwards, so that the loads of the block are in flight together.
    {
      f32x4 rk[TPG], rq[TPG], rg[TPG], rb[TPG];
      float rgs[TPG], rbe[TPG], rl[TPG];
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        const int tt = grp + NG * u;
        const size_t tok = seq0 + (size_t)min(t0 + tt, T - 1) * H;
        rk[u] = ld4x(kg + tok * DK + c4);
        rq[u] = ld4x(qg + tok * DK + c4);
        if (decay == 2) rg[u] = ld4x(p.g + tok * DK + c4);
        rgs[u] = gsrc[tok];
        if (erase == 1) rb[u] = ld4x(p.b + tok * DK + c4);
        rbe[u] = bsrc[tok];
        rl[u] = qmix == 2 ? p.lam[tok] : (qmix ? p.lam[hh] : 0.f);
      }
#pragma unroll
      for (int u = 0; u < TPG; ++u) {
        const int tt = grp + NG * u;
        const bool ok = tt < nt;
        f32x4 a, e, kk, qq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kk[i] = ok ? rk[u][i] : 0.f;
          qq[i] = ok ? rq[u][i] : 0.f;
          a[i] = !ok ? 1.f : (decay == 2 ? fexp(rg[u][i]) : (decay == 1 ? fexp(rgs[u]) : 1.f));
          if (erase == 1) e[i] = (ok ? rb[u][i] : 0.f) * kk[i];
          else if (erase == 2) e[i] = kk[i];
          else e[i] = rbe[u] * __builtin_fmaf(rl[u], qq[i], kk[i]);
        }
        *reinterpret_cast<f32x4*>(&sA[tt][c4]) = a;
        *reinterpret_cast<f32x4*>(&sE[tt][c4]) = e;
        *reinterpret_cast<f32x4*>(&sK[tt][c4]) = kk;
        *reinterpret_cast<f32x4*>(&sQ[tt][c4]) = qq;
      }
    }
    // ---- value side of my column: z, the erase multiplier m and the gate
    {
      float rv[TB], rw[TB], rgt[TB];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const size_t tok = seq0 + (size_t)min(t0 + tt, T - 1) * H;
        rv[tt] = ldx(vg + tok * DV + v);
        rw[tt] = erase == 2 ? p.beta[tok * DV + v] : (write == 1 ? p.w[tok * DV + v] : bsrc[tok]);
        rgt[tt] = epi ? ldx(gateg + tok * DV + v) : 0.f;
      }
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const bool ok = tt < nt;
        sM[tt][v] = (erase == 2 && ok) ? rw[tt] : 1.f;
        sZ[tt][v] = ok ? rw[tt] * rv[tt] : 0.f;
        sGt[tt][v] = ok ? rgt[tt] : 0.f;
      }
    }
    __syncthreads();
    float ob[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      ob[tt] = 0.f;
      if (tt < nt) {
        // forget (no decay: alpha = 1), then predict along e
        if (decay != 0) {
#pragma unroll
          for (int c = 0; c < DH; c += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(&sA[tt][cb + c]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              S[0][c + u] *= a[u];
              S[1][c + u] *= a[u];
            }
          }
        }
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int c = 0; c < DH; c += 4) {
          const f32x4 e = *reinterpret_cast<const f32x4*>(&sE[tt][cb + c]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            r0 = __builtin_fmaf(e[u], S[0][c + u], r0);
            r1 = __builtin_fmaf(e[u], S[1][c + u], r1);
          }
        }
        r0 = pair_sum(r0);
        r1 = pair_sum(r1);
        const float d0 = sZ[tt][col0] - sM[tt][col0] * r0;
        const float d1 = sZ[tt][col0 + 1] - sM[tt][col0 + 1] * r1;
        // write along k, then read along q
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int c = 0; c < DH; c += 4) {
          const f32x4 kk = *reinterpret_cast<const f32x4*>(&sK[tt][cb + c]);
          const f32x4 qq = *reinterpret_cast<const f32x4*>(&sQ[tt][cb + c]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            S[0][c + u] = __builtin_fmaf(kk[u], d0, S[0][c + u]);
            S[1][c + u] = __builtin_fmaf(kk[u], d1, S[1][c + u]);
            o0 = __builtin_fmaf(qq[u], S[0][c + u], o0);
            o1 = __builtin_fmaf(qq[u], S[1][c + u], o1);
          }
        }
        o0 = pair_sum(o0);
        o1 = pair_sum(o1);
        ob[tt] = hf ? o1 : o0;  // column v
      }
    }
    if (epi) {
      // mean of o^2 over the dv columns of each token: wave sums, then the waves'
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const float s = wave_sum(ob[tt] * ob[tt]);
        if ((v & 63) == 0) sP[tt][wave] = s;
      }
    }
    __syncthreads();  // the block's key-side vectors (and partial sums) are read
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      if (tt < nt) {
        const size_t tok = seq0 + (size_t)(t0 + tt) * H;
        float y = ob[tt];
        if (epi) {
          float ss = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) ss += sP[tt][w2];
          y = y * rsqrtf(ss * (1.f / DV) + p.eps) * nwv * silu(sGt[tt][v]);
        }
        og[tok * DV + v] = (IO)y;
      }
    }
  }
  if (p.state_out) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < DH; ++c) p.state_out[((size_t)bh * DK + cb + c) * DV + col0 + j] = S[j][c];
  }
}

// Standalone epilogue over `rows` rows of dv values (o and gate [rows][dv],
// io dtype; y may be o itself).  L lanes share one row, each with 16 bytes
// of it; 64 / L rows per wave, 4 waves per workgroup.
template <class IO, int DV>
__global__ __launch_bounds__(256) void norm_gate_kernel(const IO* o, const IO* gate, const float* nw, IO* y,
                                                        int64_t rows, float eps) {
  constexpr int EPL = 16 / sizeof(IO);  // elements per lane
  constexpr int L = DV / EPL;           // lanes per row
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "epilogue layout");
  constexpr int RPW = 64 / L;           // rows per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / L, li = lane - sub * L;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * RPW + sub;
  const bool ok = row < rows;
  const int64_t base = (ok ? row : 0) * DV + li * EPL;
  float x[EPL], gg[EPL];
  if constexpr (sizeof(IO) == 2) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + base);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(gate + base);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      x[i] = (float)a[i];
      gg[i] = (float)b[i];
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(o + base);
    const f32x4 b = *reinterpret_cast<const f32x4*>(gate + base);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      x[i] = a[i];
      gg[i] = b[i];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s = __builtin_fmaf(x[i], x[i], s);
#pragma unroll
  for (int m = 1; m < L; m <<= 1) s += __shfl_xor(s, m, L);
  const float inv = rsqrtf(s * (1.f / DV) + eps);
  float out[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) out[i] = x[i] * inv * nw[li * EPL + i] * silu(gg[i]);
  if (ok) {
    if constexpr (sizeof(IO) == 2) {
      st8(y + base, out);
    } else {
      *reinterpret_cast<f32x4*>(y + base) = f32x4{out[0], out[1], out[2], out[3]};
    }
  }
}

}  // namespace gdr
