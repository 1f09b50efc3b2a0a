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
// One workgroup per (batch, head) with dk threads.  Thread (group, l) keeps
// the state entries of key channels 16 l .. 16 l + 15 and of the dv / 16
// value columns of its column group in registers for the whole call; the
// dk / 16 lanes of a column group are consecutive, so the contractions over
// the key channels (r and o) end in a DPP sum over 4 or 8 lanes, and every
// LDS read of a staged key-side vector feeds dv / 16 columns.  The key-side
// vectors (e, k, q, one fold factor) of a block of TB = 8 tokens are staged
// in LDS by one thread per key channel, the value side (z, m, gate) by one
// thread per value column; a token needs no barrier.
//
// The decay is applied lazily: per key channel the state is held as
// s * S~, with s the product of the channel's decays since its last fold,
// so the staging scales e and q by s and k by 1/s and the token loop does no
// decay multiply.  A channel whose s would leave [2^-40, 2^40] folds s into
// its state row at that token (one multiply of the row, flagged per token),
// and the call ends with a fold of every channel.  The rounding therefore
// depends on where a sequence is split between calls (within fp32 rounding
// of the one-call result).
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

// DPP read of a neighbouring lane's value: quad_perm [1,0,3,2] (lane ^ 1),
// quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (lane i of each 8-lane
// half-row from lane 7 - i)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppX1 = 0xB1, kDppX2 = 0x4E, kDppHalfMirror = 0x141;

// sum over the G consecutive lanes (G = 4 or 8, aligned) that share a value
// column group; every lane of the group gets the sum
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<kDppX1>(x);
  x += dpp_f<kDppX2>(x);
  if constexpr (G == 8) x += dpp_f<kDppHalfMirror>(x);
  return x;
}

// one halving step of a reduce-scatter over a lane pair: the lane with `up`
// set keeps the upper half of the first L values, its partner the lower
// half, and each adds the partner's copy of the half it keeps (L = 1: plain
// sum)
template <int L, int CTRL, int N>
__device__ __forceinline__ void halve(float (&x)[N], bool up) {
  if constexpr (L == 1) {
    x[0] += dpp_f<CTRL>(x[0]);
  } else {
#pragma unroll
    for (int j = 0; j < L / 2; ++j) {
      const float keep = up ? x[j + L / 2] : x[j];
      const float send = up ? x[j] : x[j + L / 2];
      x[j] = keep + dpp_f<CTRL>(send);
    }
  }
}

template <class IO, int DK, int DV>
__global__ __launch_bounds__(DK * DV / 64) __attribute__((amdgpu_waves_per_eu(4))) void recur_fwd_kernel(RecurParams p) {
  constexpr int TB = 8;                  // tokens staged per block
  constexpr int DC = 16;                 // key channels per thread
  constexpr int G = DK / DC;             // lanes per value-column group (4 or 8)
  constexpr int NC = 4;                  // value columns per thread
  constexpr int NT = DK * DV / 64;       // threads: G lanes per group of NC columns
  constexpr int NW = NT / 64;            // waves
  constexpr int GS = DC + 4;             // padded stride of one lane's channels in a key-side row
  constexpr int RS = G * GS;             // key-side row (floats)
  constexpr int L0 = G == 8 ? (NC > 1 ? NC / 2 : 1) : NC;  // values left after the half-mirror step
  constexpr int L1 = L0 > 1 ? L0 / 2 : 1;                  // after the lane ^ 2 step
  constexpr int NO = L1 > 1 ? L1 / 2 : 1;                  // after the lane ^ 1 step: my outputs
  static_assert((G == 4 || G == 8) && NT % 64 == 0, "recurrent layout");
  __shared__ __attribute__((aligned(16))) float sE[TB][RS], sK[TB][RS], sQ[TB][RS], sF[TB][RS];
  __shared__ __attribute__((aligned(16))) float sZ[TB][DV], sM[TB][DV];
  __shared__ float sP[TB][NW];
  __shared__ float sScale[DK];
  __shared__ unsigned sFold[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % G, cgi = tid / G;   // lane in its column group, column group
  const int cb = li * DC, col0 = cgi * NC;  // my key channels and value columns
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

  // my output columns after the reduce-scatter (lanes with an odd li repeat
  // their partner's column when NC < G and do not store)
  int ocol = 0;
  {
    int L = NC;
    if constexpr (G == 8) {
      if (L > 1) { L /= 2; ocol += (li & 4) ? L : 0; }
    }
    if (L > 1) { L /= 2; ocol += (li & 2) ? L : 0; }
    if (L > 1) { L /= 2; ocol += (li & 1) ? L : 0; }
  }
  const bool ostore = NC >= G || (li & 1) == 0;
  float nwv[NO];
#pragma unroll
  for (int u = 0; u < NO; ++u) nwv[u] = epi ? p.nw[col0 + ocol + u] : 0.f;

  // S[i][j] = state row cb + i, column col0 + j, divided by the running
  // decay of channel cb + i (see below)
  float S[DC][NC];
#pragma unroll
  for (int i = 0; i < DC; ++i)
#pragma unroll
    for (int j4 = 0; j4 < NC / 4; ++j4) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p.state_in) x = *reinterpret_cast<const f32x4*>(p.state_in + ((size_t)bh * DK + cb + i) * DV + col0 + 4 * j4);
#pragma unroll
      for (int u = 0; u < 4; ++u) S[i][4 * j4 + u] = x[u];
    }
  if (tid == 0) sFold[0] = sFold[1] = 0u;
  __syncthreads();

  // Staging: thread c owns key channel c.  The decay is applied lazily: the
  // state is kept as Diag(s) S~ with s the product of the channel's decays
  // since the last fold, so a token's decay costs nothing in the token loop;
  // e and q are staged times s and k divided by s.  When s of some channel
  // would leave [2^-40, 2^40] at a token (a strong decay, or a decay of
  // exactly zero), that token folds: the staging writes the factor f = s for
  // the channel, the token loop multiplies the channel's state row by it and
  // s restarts at 1.  The call ends with one fold of every channel.
  const int c = tid;                      // key-side staging: threads c < DK
  const bool kside = c < DK;
  const int ci = (c / DC) * GS + c % DC;  // channel c in a key-side row
  const int vt = (tid + NT - DK) % NT;    // value-side staging: from thread DK on
  float srun = 1.f;
  // (a readable stand-in where beta is absent: its loads are never used)
  const float* bsrc = (erase == 0 || write == 0) ? p.beta : reinterpret_cast<const float*>(p.v);
  for (int t0 = 0, blk = 0; t0 < T; t0 += TB, ++blk) {
    const int nt = min(TB, T - t0);
    if (tid == 0) sFold[(blk + 1) & 1] = 0u;  // flags of the next block (last read two barriers ago)
    if (kside) {
      // the loads of four tokens at a time first, at token indices clamped
      // to T - 1; each array is addressed from the block's first token with
      // 32-bit offsets, so that the loads take the scalar-base form
      const size_t row0 = seq0 + (size_t)t0 * H;  // token row of the block's first token
      const IO* kb = kg + row0 * DK;
      const IO* qb = qg + row0 * DK;
      const float* gb = decay == 2 ? p.g + row0 * DK : p.g + row0;
      const float* bb_ = erase == 1 ? p.b + row0 * DK : nullptr;
      const float* beb = bsrc + row0;
      const float* lb = qmix == 2 ? p.lam + row0 : nullptr;
      unsigned fold = 0u;
#pragma unroll
      for (int h = 0; h < TB; h += 4) {
        float kx[4], qx[4], gx[4], bx[4], bex[4], lx[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const unsigned r = (unsigned)min(h + u, nt - 1) * (unsigned)H;  // token row within the block
          kx[u] = ldx(kb + (r * DK + c));
          qx[u] = ldx(qb + (r * DK + c));
          gx[u] = decay == 2 ? gb[r * DK + c] : (decay == 1 ? gb[r] : 0.f);
          bx[u] = erase == 1 ? bb_[r * DK + c] : 0.f;
          bex[u] = beb[r];
          lx[u] = qmix == 2 ? lb[r] : (qmix ? p.lam[hh] : 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int tt = h + u;
          const bool ok = tt < nt;
          float kk = ok ? kx[u] : 0.f, qq = ok ? qx[u] : 0.f;
          float e;
          if (erase == 1) e = bx[u] * kk;
          else if (erase == 2) e = kk;
          else e = bex[u] * __builtin_fmaf(lx[u], qq, kk);
          float f = 1.f;
          if (decay != 0) {
            float sp = srun * (ok ? fexp(gx[u]) : 1.f);
            if (!(sp >= 0x1p-40f && sp <= 0x1p40f)) {
              f = sp;
              sp = 1.f;
              fold |= 1u << tt;
            }
            srun = sp;
            e *= sp;
            qq *= sp;
            kk *= __builtin_amdgcn_rcpf(sp);
          }
          sE[tt][ci] = e;
          sK[tt][ci] = kk;
          sQ[tt][ci] = qq;
          sF[tt][ci] = f;
        }
      }
      if (fold) atomicOr(&sFold[blk & 1], fold);
    }
    // value side: column vt, vt + NT, ... (z and the erase multiplier m)
#pragma unroll 1
    for (int vc = vt; vc < DV; vc += NT) {
      const size_t row0 = seq0 + (size_t)t0 * H;
      const IO* vb = vg + row0 * DV + vc;
      const float* wb = erase == 2 ? p.beta + row0 * DV + vc : (write == 1 ? p.w + row0 * DV + vc : nullptr);
      const float* beb = bsrc + row0;
      float rv[TB], rw[TB];
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const unsigned r = (unsigned)min(tt, nt - 1) * (unsigned)H;
        rv[tt] = ldx(vb + r * DV);
        rw[tt] = (erase == 2 || write == 1) ? wb[r * DV] : beb[r];
      }
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const bool ok = tt < nt;
        sM[tt][vc] = (erase == 2 && ok) ? rw[tt] : 1.f;
        sZ[tt][vc] = ok ? rw[tt] * rv[tt] : 0.f;
      }
    }
    __syncthreads();

    // token loop: r = S_bar^T e, d = z - m (.) r, S += k d^T, o = S^T q, with
    // the contractions over my 16 channels and then over the G lanes
    const unsigned fb = sFold[blk & 1];
    float ob[TB][NO];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
#pragma unroll
      for (int u = 0; u < NO; ++u) ob[tt][u] = 0.f;
      if (tt < nt) {
        if (fb & (1u << tt)) {
#pragma unroll
          for (int i4 = 0; i4 < DC / 4; ++i4) {
            const f32x4 f = *reinterpret_cast<const f32x4*>(&sF[tt][li * GS + 4 * i4]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int j = 0; j < NC; ++j) S[4 * i4 + u][j] *= f[u];
          }
        }
        float r[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) r[j] = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < DC / 4; ++i4) {
          const f32x4 e = *reinterpret_cast<const f32x4*>(&sE[tt][li * GS + 4 * i4]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NC; ++j) r[j] = __builtin_fmaf(e[u], S[4 * i4 + u][j], r[j]);
        }
        float d[NC];
#pragma unroll
        for (int j4 = 0; j4 < NC / 4; ++j4) {
          const f32x4 z = *reinterpret_cast<const f32x4*>(&sZ[tt][col0 + 4 * j4]);
          f32x4 m = f32x4{1.f, 1.f, 1.f, 1.f};
          if (erase == 2) m = *reinterpret_cast<const f32x4*>(&sM[tt][col0 + 4 * j4]);
#pragma unroll
          for (int u = 0; u < 4; ++u) d[4 * j4 + u] = z[u] - m[u] * group_sum<G>(r[4 * j4 + u]);
        }
        float o[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) o[j] = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < DC / 4; ++i4) {
          const f32x4 kk = *reinterpret_cast<const f32x4*>(&sK[tt][li * GS + 4 * i4]);
          const f32x4 qq = *reinterpret_cast<const f32x4*>(&sQ[tt][li * GS + 4 * i4]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NC; ++j) {
              S[4 * i4 + u][j] = __builtin_fmaf(kk[u], d[j], S[4 * i4 + u][j]);
              o[j] = __builtin_fmaf(qq[u], S[4 * i4 + u][j], o[j]);
            }
        }
        // reduce-scatter of o over the G lanes: lane li ends with columns
        // ocol .. ocol + NO - 1
        if constexpr (G == 8) halve<NC, kDppHalfMirror>(o, (li & 4) != 0);
        halve<L0, kDppX2>(o, (li & 2) != 0);
        halve<L1, kDppX1>(o, (li & 1) != 0);
#pragma unroll
        for (int u = 0; u < NO; ++u) ob[tt][u] = o[u];
      }
    }
    if (epi) {
      // mean of o^2 over the dv columns of each token: wave sums, then the waves'
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        float s2 = 0.f;
#pragma unroll
        for (int u = 0; u < NO; ++u) s2 += ob[tt][u] * ob[tt][u];
        const float s = wave_sum(ostore ? s2 : 0.f);
        if (lane == 0) sP[tt][wave] = s;
      }
    }
    __syncthreads();  // the block's staged vectors (and partial sums) are read
    if (ostore) {
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        if (tt < nt) {
          const size_t tok = seq0 + (size_t)(t0 + tt) * H;
          float inv = 1.f;
          if (epi) {
            float ss = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) ss += sP[tt][w2];
            inv = rsqrtf(ss * (1.f / DV) + p.eps);
          }
#pragma unroll
          for (int u = 0; u < NO; ++u) {
            const int col = col0 + ocol + u;
            float y = ob[tt][u];
            if (epi) y = y * inv * nwv[u] * silu(ldx(gateg + tok * DV + col));
            og[tok * DV + col] = (IO)y;
          }
        }
      }
    }
  }
  if (p.state_out) {
    if (decay != 0) {
      // the closing fold: S = Diag(s) S~
      if (kside) sScale[c] = srun;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < DC; ++i) {
        const float f = sScale[cb + i];
#pragma unroll
        for (int j = 0; j < NC; ++j) S[i][j] *= f;
      }
    }
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int j4 = 0; j4 < NC / 4; ++j4)
        *reinterpret_cast<f32x4*>(p.state_out + ((size_t)bh * DK + cb + i) * DV + col0 + 4 * j4) =
            f32x4{S[i][4 * j4], S[i][4 * j4 + 1], S[i][4 * j4 + 2], S[i][4 * j4 + 3]};
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
