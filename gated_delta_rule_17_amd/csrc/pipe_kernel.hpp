// Pipelined chunkwise forward of the generalized gated delta rule on gfx950,
// for bf16 inputs with no decay or a per-head scalar decay and the scalar
// (beta) erase gate; the write gate may be beta or per value channel, and the
// Q-Delta mix x = k + lambda q is supported.
//
// Same chunk algebra as chunk_kernel.hpp (the chunk WY form with absorbed
// decay of "Gated DeltaNet-2: Decoupling Erase and Write in Linear
// Attention", key design 2), regrouped so that only three small products
// depend on the state:
//   T   = tril(diag(beta gamma) E K^T diag(1/gamma), -1),  A = (I + T)^{-1}
//   A_qk = tril(diag(gamma) Q K^T diag(1/gamma), 0)
//   W   = A (Z - diag(beta gamma) E S)          (= U - Y S of the page)
//   O   = diag(gamma) Q S + A_qk W
//   S'  = gamma_C S + K^T diag(tail) W,          tail_j = gamma_C / gamma_j
// with E = K, or K + lambda Q under the Q-Delta mix.  The per-token scalars
// scale accumulator rows, so K and Q enter the MFMAs as the raw bf16 inputs
// and the decay ratios are formed as exp(G_i - G_j) <= 1.
//
// Workgroup = NCW consumer waves (two, or one for a 16-column slice) + 4
// producer waves.  At step i
// the producers turn chunk i into LDS operands (inputs, Gram, A = (I+T)^-1)
// while the consumers apply chunk i - 1 to the state.  Every per-chunk LDS
// buffer is double-buffered; each step has three workgroup barriers:
//   phase 1  producers: rows of k, q, v and the chunk     | consumers: K S, Q S
//            scalars to LDS
//   phase 2  producers: T and A_qk tiles (MFMA)            | consumers: W, O to LDS
//   phase 3  producer waves 0, 1: A = (I + T)^{-1}         | consumers: S update, O stores
//
// Consumer wave c owns 32 value columns of a 64-column slice (16 of a
// narrower one) and all DK rows of the state, in MFMA accumulators.  Products whose contraction
// index is the accumulator row index take the accumulator (converted to
// bf16) directly as an MFMA operand; the k order that this imposes is
// matched on the LDS side, by the choice of rows in row reads and of rows and
// column groups in transposing reads (ds_read_b64_tr_b16).  State tile 2m+h,
// accumulator row 4g+r (g = lane / 16) holds channel 32m + 8g + 4h + r.
#pragma once

#include "chunk_kernel.hpp"
#include "common.hpp"

namespace gdr {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16.  In each group of 16 lanes, lane s gives the address of
// row s / 4, columns 4 (s % 4) .. +3 of a 4 x 16 block of 16-bit values; lane
// i receives column i of the block (rows 0..3).  Each group has its own block.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x4 cvt4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f32x4 cvtf4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x16: A/B fragment of lane l = 4 consecutive k (k = 4 (l / 16) .. +3)
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                  0, 0, 0);
}

// The (I, J) 16x16 tiles of T and A_qk that one producer wave computes.
template <int N_, int I0, int J0, int I1, int J1, int I2 = 0, int J2 = 0>
struct Tiles {
  static constexpr int n = N_;
  static constexpr int I(int t) { return t == 0 ? I0 : (t == 1 ? I1 : I2); }
  static constexpr int J(int t) { return t == 0 ? J0 : (t == 1 ? J1 : J2); }
};

// Forward substitution x <- (I + T)^{-1} x for a 16 x 16 strictly lower T
// whose row i sits in lane i of each 16-lane row (tr = its 16 floats): for
// j = 0..14 and i > j, x[i] += T[i][j] (-x[j]), with T[i][j] broadcast from
// lane i by the DPP row_newbcast:i operand of one v_fmac_f32.  The s_nop
// before the first use of a column gives the two wait states that a DPP
// source needs after a VALU write.
template <int J, int I>
__device__ __forceinline__ void subst_col(float (&x)[16], float tj, float nxj) {
  if constexpr (I < 16) {
    if constexpr (I == J + 1)
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(x[I])
                   : "v"(tj), "v"(nxj), "n"(I));
    else
      asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(x[I])
                   : "v"(tj), "v"(nxj), "n"(I));
    subst_col<J, I + 1>(x, tj, nxj);
  }
}
template <int J>
__device__ __forceinline__ void subst(float (&x)[16], const float (&tr)[16]) {
  if constexpr (J < 15) {
    subst_col<J, J + 1>(x, tr[J], -x[J]);
    subst<J + 1>(x, tr);
  }
}

// A = (I + T)^{-1} for the 64 x 64 strictly lower T of a chunk, on one wave.
// T's four diagonal 16x16 blocks come as fp32 rows (block b, row i at
// Td + b TDB + i TDS), the blocks below the diagonal as bf16 rows of Tm (row
// stride SC); A goes to Ab column-major (Ab[j SC + i] = A[i][j]), whose blocks
// above the diagonal must already be zero.
//   level 0: lane (block g, column l16) forward-substitutes column l16 of
//            (I + T_gg)^{-1}; lane i of each 16-lane row holds row i of T_gg
//   level 1: A_IJ = -A_II (T_IJ A_JJ) for (I, J) = (1, 0), (3, 2)
//   level 2: P_IJ = T[I, 0:32] A[0:32, J], A_IJ = -A[I, 32:64] P[32:64, J]
// JM selects the level-2 column blocks J (bit J) that this call forms: two
// waves can split level 2, each redoing levels 0 and 1 (their identical
// writes of those blocks are harmless, and each wave reads them only after
// writing them itself).
template <int SC, int TDS, int TDB, int JM = 3>
__device__ __forceinline__ void solve_inverse(const float* Td, const bf16* Tm, bf16* Ab, int g, int l16) {
  float tr[16];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(Td + g * TDB + l16 * TDS + 4 * q4);
#pragma unroll
    for (int e = 0; e < 4; ++e) tr[4 * q4 + e] = v[e];
  }
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (i == l16) ? 1.f : 0.f;
  subst<0>(x, tr);
  st8(Ab + (16 * g + l16) * SC + 16 * g, x);
  st8(Ab + (16 * g + l16) * SC + 16 * g + 8, x + 8);

  // level 1: A_IJ = -A_II (T_IJ A_JJ) for (I, J) = (1, 0), (3, 2)
  f32x4 P1[2];
#pragma unroll
  for (int bp = 0; bp < 2; ++bp) {
    const int I = 2 * bp + 1, J = 2 * bp;
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(Tm + (16 * I + l16) * SC + 16 * J + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(Ab + (16 * J + l16) * SC + 16 * J + 4 * g);
    P1[bp] = mma16(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int bp = 0; bp < 2; ++bp) {
    const int I = 2 * bp + 1, J = 2 * bp;
    const bf16x4 a = lds_tr4(Ab + (16 * I + 4 * g + (l16 >> 2)) * SC + 16 * I + 4 * (l16 & 3));
    const f32x4 r = mma16(a, cvt4(P1[bp]), f32x4{0.f, 0.f, 0.f, 0.f});
    *reinterpret_cast<bf16x4*>(Ab + (16 * J + l16) * SC + 16 * I + 4 * g) = cvt4(-r);
  }
  // level 2: P_IJ = T[I, 0:32] A[0:32, J], A_IJ = -A[I, 32:64] P[32:64, J]
  f32x4 P2[2][2];
#pragma unroll
  for (int I = 2; I < 4; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) {
      if (!((JM >> J) & 1)) continue;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Tm + (16 * I + l16) * SC + 8 * g);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Ab + (16 * J + l16) * SC + 8 * g);
      P2[I - 2][J] = mma32(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
  for (int I = 2; I < 4; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) {
      if (!((JM >> J) & 1)) continue;
      const bf16x4 a1 = lds_tr4(Ab + (32 + 4 * g + (l16 >> 2)) * SC + 16 * I + 4 * (l16 & 3));
      const bf16x4 a2 = lds_tr4(Ab + (48 + 4 * g + (l16 >> 2)) * SC + 16 * I + 4 * (l16 & 3));
      const f32x4 r = mma32(cat8(a1, a2), cat8(cvt4(P2[0][J]), cvt4(P2[1][J])), f32x4{0.f, 0.f, 0.f, 0.f});
      *reinterpret_cast<bf16x4*>(Ab + (16 * J + l16) * SC + 16 * I + 4 * g) = cvt4(-r);
    }
}

// Stored triangles: a [64][64] bf16 matrix whose six 16 x 16 blocks above
// (or below) the diagonal are zero keeps only its ten other blocks, as 320
// pieces of 16 bytes.  Lower: row block I holds its blocks J <= I, rows of
// 32 (I + 1) bytes, row blocks in order.  Upper: row block J holds its
// blocks I >= J, rows of 32 (4 - J) bytes.
// Piece q (< 320) of a stored triangle -> (row, 16-byte column) of the dense
// matrix.
struct TriPiece {
  int row, col;
};
__device__ __forceinline__ TriPiece tri_lower_piece(int q) {
  const int I = q < 32 ? 0 : q < 96 ? 1 : q < 192 ? 2 : 3;
  const int w = 2 * (I + 1), l = q - 16 * I * (I + 1);
  return {16 * I + l / w, l % w};
}
__device__ __forceinline__ TriPiece tri_upper_piece(int q) {
  const int J = q < 128 ? 0 : q < 224 ? 1 : q < 288 ? 2 : 3;
  const int w = 2 * (4 - J), l = q - (J == 0 ? 0 : J == 1 ? 128 : J == 2 ? 224 : 288);
  return {16 * J + l / w, 2 * J + l % w};
}
// Byte offset, within a stored lower triangle, of row r of the dense matrix at
// bf16 column c (c in a block J <= r / 16).
__device__ __forceinline__ int tri_lower_byte(int r, int c) {
  const int I = r >> 4;
  return 512 * (I * (I + 1) / 2) + 32 * (I + 1) * (r & 15) + 2 * c;
}

// T and A_qk tiles (list TL) of one chunk under no or a scalar decay, as
// D^T = K_J X_I^T (X = K, or K + lam Q under the Q-Delta mix, for T; Q for
// A_qk), so that each lane holds four consecutive columns j of one row i;
// then the decay exp(G_i - G_j) <= 1, beta_i on T, and the masks (T: j < i,
// A_qk: j <= i).  K, Q rows of strides SK, SQ; G and beta per token.  T below
// the diagonal blocks goes to bf16 rows of sT (stride SC), its diagonal
// blocks to fp32 rows of sTd (block stride TDB, row stride TDS); A_qk to bf16
// rows of aqk with row stride AS, or (TRI) to aqk as a stored lower triangle.
template <int DK, int SK, int SQ, int SC, int TDS, int TDB, bool MIX, bool TRI = false, class TL>
__device__ __forceinline__ void scalar_gram_tiles(TL, const bf16* Kb, const bf16* Qb, const float* sG,
                                                  const float* sBeta, float lam, bf16* sT, float* sTd, bf16* aqk,
                                                  int AS, int g, int l16) {
  constexpr int NT = TL::n, NKS = DK / 32;
  // fragments of 16 rows (identical loads are merged by the compiler)
  auto kfr = [&](int blk, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(Kb + (16 * blk + l16) * SK + 32 * s + 8 * g);
  };
  auto qfr = [&](int blk, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(Qb + (16 * blk + l16) * SQ + 32 * s + 8 * g);
  };
  f32x4 accT[NT], accA[NT];
  float Gi[NT], bi[NT];
  f32x4 Gj[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int I = TL::I(t), J = TL::J(t);
    Gi[t] = sG[16 * I + l16];
    bi[t] = sBeta[16 * I + l16];
    Gj[t] = *reinterpret_cast<const f32x4*>(sG + 16 * J + 4 * g);
    accT[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    accA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 kj = kfr(J, s), ki = kfr(I, s), qi = qfr(I, s);
      bf16x8 xi = ki;
      if constexpr (MIX) {
#pragma unroll
        for (int c = 0; c < 8; ++c) xi[c] = (bf16)((float)ki[c] + lam * (float)qi[c]);
      }
      accT[t] = mma32(kj, xi, accT[t]);
      accA[t] = mma32(kj, qi, accA[t]);
    }
  }
  // decay, beta and masks; i = row (lane), j = 4 columns
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int I = TL::I(t), J = TL::J(t);
    const int i = 16 * I + l16, j0 = 16 * J + 4 * g;
    f32x4 xT, xA;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fexp(Gi[t] - Gj[t][r]);
      xT[r] = (j0 + r < i) ? bi[t] * accT[t][r] * e : 0.f;  // T: j < i
      xA[r] = (j0 + r <= i) ? accA[t][r] * e : 0.f;         // A_qk: j <= i
    }
    if constexpr (TRI) *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(aqk) + tri_lower_byte(i, j0)) = cvt4(xA);
    else *reinterpret_cast<bf16x4*>(aqk + i * AS + j0) = cvt4(xA);
    if (J < I) *reinterpret_cast<bf16x4*>(sT + i * SC + j0) = cvt4(xT);
    else *reinterpret_cast<f32x4*>(sTd + I * TDB + l16 * TDS + 4 * g) = xT;
  }
}

// ---- LDS layout (byte offsets) -------------------------------------------
template <int DK, int DVS, bool KT = false>
struct PipeLay {
  // Row strides (bf16 elements), chosen from measured LDS bank conflicts
  // on gfx950 (64 four-byte banks) for each array's own access patterns:
  //   k: 16-row b128 fragment reads and transposing reads of rows 8g + l/4
  //      pull in opposite directions; 320 B rows give the least in total
  //   q: b128 fragment reads only; 288 B (dk 128) and 160 B rows are free
  //   Z: transposing reads of rows 4g + l/4; 160 B rows (64 columns) are free
  //   O staging: b64 writes of 16 rows x 4 groups; 136 B rows are free
  //   K^T (record mode): b128 reads of channels 8a + b (a, b < 4) of one
  //      16-token run; 144 B rows with the run index XORed with 4 in
  //      channels 16..31 of every 32 are free (see kt_off)
  static constexpr int SK = DK + (DK == 128 ? 32 : 24);  // k rows: 320 B (dk 128) / 176 B (dk 64)
  static constexpr int SQ = DK + 16;         // q rows
  static constexpr int SC = CH + 8;          // bf16 row stride of the [64][64] arrays
  static constexpr int SZ = DVS == 64 ? 80 : DVS + 8;  // bf16 row stride of Z
  static constexpr int TDS = 20;             // fp32 row stride inside a diagonal T block
  static constexpr int TDB = 16 * TDS;       // fp32 stride between the four diagonal blocks
  // per-chunk scalars (float offsets): G = chunk cumsum of the log-decay,
  // beta, c_e = beta gamma, gamma, tail = gamma_C / gamma, gamma_C
  static constexpr int sG = 0, sBeta = 64, sCE = 128, sGam = 192, sTail = 256, sGC = 320, NSC = 336;
  static constexpr int SO = CH + 4;          // O staging: [DVS][64] (value column, token)
  static constexpr int szK = CH * SK * 2, szQ = CH * SQ * 2, szZ = CH * SZ * 2, szA = CH * SC * 2, szS = NSC * 4;
  static constexpr int oK = 0;                 // 2 x [64][SK]  k rows (zero past the end)
  static constexpr int oQ = oK + 2 * szK;      // 2 x [64][SQ]  q rows
  static constexpr int oZ = oQ + 2 * szQ;      // [64][SZ]  gated v rows: beta * v or w * v (written
                                               // and read in the same step)
  static constexpr int oAcm = oZ + szZ;        // 2 x [64][SC]  A column-major: Acm[j][i] = A[i][j]
  static constexpr int oAqk = oAcm + 2 * szA;  // 2 x [64][SC]  A_qk row-major
  static constexpr int oSc = oAqk + 2 * szA;   // 2 x scalars
  static constexpr int oT = oSc + 2 * szS;     // [64][SC] T row-major, blocks below the diagonal (producers)
  static constexpr int oTd = oT + szA;         // 4 x [16][TDS] fp32: Td[b][i][j] = T[16b+i][16b+j] (producers)
  static constexpr int oO = oTd + 4 * TDB * 4;  // [DVS][SO] output staging (consumers)
  static constexpr int oKT = oO + DVS * SO * 2;  // record mode: [DK][SKT] K^T (channel, token)
  static constexpr int SKT = CH + 8;
  static constexpr int TOTAL = oKT + (KT ? DK * SKT * 2 : 0);
  static_assert(TOTAL <= 160 * 1024, "LDS budget exceeded");
  static_assert(NSC == 336 && NSC % 4 == 0, "the two-pass record holds NSC scalars");
  static_assert(oQ % 16 == 0 && oZ % 16 == 0 && oAcm % 16 == 0 && oAqk % 16 == 0 && oSc % 16 == 0 &&
                    oT % 16 == 0 && oTd % 16 == 0 && oO % 16 == 0 && oKT % 16 == 0 && (SK * 2) % 16 == 0,
                "alignment");
};

// Byte offset in the K^T array (rows of SKT = 72 bf16) of the 16-byte run r
// (tokens 8r .. 8r + 7) of channel c.  A consumer fragment read takes
// channels 32m + 8a + 4h + b (a, b < 4) of one run; with 144-byte rows
// those pairs a, a + 2 hit the same banks, so the run index is XORed with 4
// in channels 16..31 of every 32.
__device__ __forceinline__ int kt_off(int c, int r) { return c * ((CH + 8) * 2) + 16 * (r ^ (((c >> 4) & 1) << 2)); }

// Workspace record of one chunk for the two-pass form (pipe_split_kernel.hpp
// writes it, pipe_fwd_kernel<..., PRE = true> reads it): A column-major and
// A_qk row-major, [64][64] bf16 each, then the NSC chunk scalars.
struct PipeRec {
  static constexpr int NSC = 336;  // PipeLay::NSC
  static constexpr int PIECES_A = 320;  // A (column-major) and A_qk as stored triangles
  static constexpr int oAcm = 0, oAqk = PIECES_A * 16, oSc = 2 * PIECES_A * 16;
  static constexpr int NPIECE = (oSc + NSC * 4) / 16;  // 16-byte pieces
  static constexpr int BYTES = (oSc + NSC * 4 + 255) / 256 * 256;
};

// consumer waves for a value slice of DVS columns: two 32-column waves for
// 64, two 16-column waves for 32, one for 16
template <int DVS>
constexpr int pipe_ncw() {
  return DVS >= 32 ? 2 : 1;
}

// PRE: the second pass of the two-pass form, whose producer waves copy each
// chunk's record (A, A_qk, scalars; pipe_split_kernel.hpp) from p.ws into LDS
// instead of forming it.
template <int DK, int DVS, int GM, bool PRE = false>
__global__ __launch_bounds__(64 * (pipe_ncw<DVS>() + 4)) void pipe_fwd_kernel(ChunkParams p) {
  constexpr int NCW = pipe_ncw<DVS>();
  constexpr int NB = DVS / (16 * NCW);  // 16-column blocks per consumer wave
  using L = PipeLay<DK, DVS, PRE>;
  constexpr int SK = L::SK, SQ = L::SQ, SC = L::SC, SZ = L::SZ, SO = L::SO, TDS = L::TDS, TDB = L::TDB,
                NSC = L::NSC;
  constexpr int NKS = DK / 32;  // 32-channel k-steps
  constexpr bool write_ch = (GM == 3);
  static_assert(GM == 0 || GM == 3, "the pipelined kernel takes the beta erase gate");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  bf16* sK = reinterpret_cast<bf16*>(smem + L::oK);
  bf16* sQ = reinterpret_cast<bf16*>(smem + L::oQ);
  bf16* sZ = reinterpret_cast<bf16*>(smem + L::oZ);
  bf16* sAcm = reinterpret_cast<bf16*>(smem + L::oAcm);
  bf16* sAqk = reinterpret_cast<bf16*>(smem + L::oAqk);
  float* sSc = reinterpret_cast<float*>(smem + L::oSc);
  bf16* sT = reinterpret_cast<bf16*>(smem + L::oT);
  float* sTd = reinterpret_cast<float*>(smem + L::oTd);
  bf16* sO = reinterpret_cast<bf16*>(smem + L::oO);
  char* sKT = smem + L::oKT;  // record mode only

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;

  // workgroup -> (batch, head, value slice); blockIdx values that share a
  // residue mod 8 run on one XCD, so the slices of a head share its L2
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
  const size_t seq0 = (size_t)bb * T * H + hh;  // token row of (bb, t = 0, hh)

  // A and A_qk: blocks above the diagonal are never written and stay zero,
  // so triangular products can run over whole 32-wide k-steps
  {
    uint4* z = reinterpret_cast<uint4*>(smem + L::oAcm);
    for (int e = tid; e < (4 * L::szA) / 16; e += 64 * (NCW + 4)) z[e] = uint4{0u, 0u, 0u, 0u};
  }

  if (wave < NCW) {
    // =================== consumers ===========================================
    // wave c owns value columns [16 NB c, 16 NB (c + 1)) of the slice as NB
    // blocks of 16; every LDS fragment serves the NB blocks.
    const int cw0 = 16 * NB * wave;  // first slice column of this wave
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

    // step 0: the producers build chunk 0
    __syncthreads();
    __syncthreads();
    __syncthreads();
    for (int n = 0; n < nchunks; ++n) {
      const int buf = n & 1;
      const bf16* Kb = sK + buf * CH * SK;
      const bf16* Qb = sQ + buf * CH * SQ;
      const bf16* Zb = sZ;
      const bf16* Ab = sAcm + buf * CH * SC;
      const bf16* Aqb = sAqk + buf * CH * SC;
      const float* sc = sSc + buf * NSC;

      // LDS fragments of the later phases: A (transposing reads: A^T rows as
      // the k slots of W's products), A_qk rows, K^T (state update).  Waves
      // of one 16-column block have registers to spare and few products to
      // hide a read behind, so they request each phase's fragments at the
      // end of the phase before (the buffers of chunk n - 1 are complete
      // since the last step and are not rewritten in this one).
      auto afrag = [&](int pp, int h, int m2) __attribute__((always_inline)) {
        const int col = 32 * pp + 8 * (l16 & 3) + 4 * h;
        return cat8(lds_tr4(Ab + (32 * m2 + 4 * g + (l16 >> 2)) * SC + col),
                    lds_tr4(Ab + (32 * m2 + 16 + 4 * g + (l16 >> 2)) * SC + col));
      };
      auto aqfrag = [&](int I, int pp) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(Aqb + (16 * I + l16) * SC + 32 * pp + 8 * g);
      };
      auto ktfrag = [&](int j, int pp) __attribute__((always_inline)) {
        if constexpr (PRE) {
          // channel 32 (j / 2) + 8 (l16 / 4) + 4 (j % 2) + l16 % 4, tokens 32 pp + 8 g ..
          const int c = 32 * (j >> 1) + 8 * (l16 >> 2) + 4 * (j & 1) + (l16 & 3);
          return *reinterpret_cast<const bf16x8*>(sKT + kt_off(c, 4 * pp + g));
        } else {
          const int col = 32 * (j >> 1) + 8 * (l16 & 3) + 4 * (j & 1);
          return cat8(lds_tr4(Kb + (32 * pp + 8 * g + (l16 >> 2)) * SK + col),
                      lds_tr4(Kb + (32 * pp + 8 * g + 4 + (l16 >> 2)) * SK + col));
        }
      };
      constexpr bool kAhead = NB == 1, kAheadA = true;
      bf16x8 Af[kAheadA ? 2 : 1][2][2], Aq[kAheadA ? 4 : 1][2], Kt[kAhead ? 2 * NKS : 1][2];

      // ---- phase 1: K S and Q S (rows = tokens) ----------------------------
      f32x4 KS[4][NB], QS[4][NB];
      {
        bf16x8 Sb[NKS][NB];  // k slots of lane group g: channels 32 m + 8 g + e
#pragma unroll
        for (int m = 0; m < NKS; ++m)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Sb[m][nb] = cat8(cvt4(S[2 * m][nb]), cvt4(S[2 * m + 1][nb]));
        // fragments of row block I + 1 are loaded while block I multiplies
        // fragments of row block I + AHEAD are requested while block I
        // multiplies; a one-block wave has fewer products to cover a read,
        // so it looks two blocks ahead
        constexpr int AHEAD = NB == 1 ? 2 : 1, RING = AHEAD + 1;
        bf16x8 kf[RING][NKS], qf[RING][NKS];
        auto load_kq = [&](int I, int slot) {
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
            kf[slot][m] = *reinterpret_cast<const bf16x8*>(Kb + (16 * I + l16) * SK + 32 * m + 8 * g);
            qf[slot][m] = *reinterpret_cast<const bf16x8*>(Qb + (16 * I + l16) * SQ + 32 * m + 8 * g);
          }
        };
#pragma unroll
        for (int I = 0; I < AHEAD; ++I) load_kq(I, I);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I + AHEAD < 4) load_kq(I + AHEAD, (I + AHEAD) % RING);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            KS[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            QS[I][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NKS; ++m) {
              KS[I][nb] = mma32(kf[I % RING][m], Sb[m][nb], KS[I][nb]);
              QS[I][nb] = mma32(qf[I % RING][m], Sb[m][nb], QS[I][nb]);
            }
          }
        }
        if constexpr (kAheadA) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int m2 = 0; m2 <= pp; ++m2) Af[pp][h][m2] = afrag(pp, h, m2);
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int pp = 0; pp <= I / 2; ++pp) Aq[I][pp] = aqfrag(I, pp);
        }
      }
      __syncthreads();

      // ---- phase 2: W = A (Z - c_e E S), O = gamma Q S + A_qk W; O to LDS ----
      // W tile 2p+h, accumulator row 4g+r holds token 32p + 8g + 4h + r
      f32x4 Wt[4][NB];
      {
        bf16x8 Rb[2][NB];  // k slots of group g: tokens 32p + 4g + e, 32p + 16 + 4g + (e - 4)
        // Z rows carry the write gate already (beta or w, applied by the producers)
        auto residual = [&](auto qm) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              f32x4 R2[2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int I = 2 * pp + h;
                const f32x4 z = cvtf4(
                    lds_tr4(Zb + (16 * I + 4 * g + (l16 >> 2)) * SZ + cw0 + 16 * nb + 4 * (l16 & 3)));
                const f32x4 ce = *reinterpret_cast<const f32x4*>(sc + L::sCE + 16 * I + 4 * g);
                f32x4 es = KS[I][nb];
                if constexpr (decltype(qm)::value) es += lam * QS[I][nb];
                R2[h] = z - ce * es;
              }
              Rb[pp][nb] = cat8(cvt4(R2[0]), cvt4(R2[1]));
            }
        };
        if (qmix) residual(IC<1>{});
        else residual(IC<0>{});
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m2 = 0; m2 <= pp; ++m2) {
              bf16x8 af;
              if constexpr (kAheadA) af = Af[pp][h][m2];
              else af = afrag(pp, h, m2);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) acc[nb] = mma32(af, Rb[m2][nb], acc[nb]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) Wt[2 * pp + h][nb] = acc[nb];
          }
        bf16x8 Wb[2][NB];  // k slots of group g: tokens 32p + 8g + e
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) Wb[pp][nb] = cat8(cvt4(Wt[2 * pp][nb]), cvt4(Wt[2 * pp + 1][nb]));
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const f32x4 gm = *reinterpret_cast<const f32x4*>(sc + L::sGam + 16 * I + 4 * g);
          f32x4 acc[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[nb] = gm * QS[I][nb];
#pragma unroll
          for (int pp = 0; pp <= I / 2; ++pp) {
            bf16x8 af;
            if constexpr (kAheadA) af = Aq[I][pp];
            else af = aqfrag(I, pp);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = mma32(af, Wb[pp][nb], acc[nb]);
          }
          // staging is [value column][token]: 4 consecutive tokens per lane
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            *reinterpret_cast<bf16x4*>(sO + (cw0 + 16 * nb + l16) * SO + 16 * I + 4 * g) = cvt4(acc[nb]);
        }
        if constexpr (kAhead) {
#pragma unroll
          for (int j = 0; j < 2 * NKS; ++j)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) Kt[j][pp] = ktfrag(j, pp);
        }
      }
      __syncthreads();

      // ---- phase 3: S = gamma_C S + K^T diag(tail) W; outputs ---------------
      {
        const float gC = sc[L::sGC];
        bf16x8 Wtb[2][NB];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(sc + L::sTail + 32 * pp + 8 * g);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(sc + L::sTail + 32 * pp + 8 * g + 4);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            Wtb[pp][nb] = cat8(cvt4(t0 * Wt[2 * pp][nb]), cvt4(t1 * Wt[2 * pp + 1][nb]));
        }
        // transposed K fragments of state tile j + 1 are loaded while tile j
        // multiplies (one-block waves have all of them already)
        bf16x8 kt[2][2];
        auto load_kt = [&](int j, int slot) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) kt[slot][pp] = ktfrag(j, pp);
        };
        if constexpr (!kAhead) load_kt(0, 0);
#pragma unroll
        for (int j = 0; j < 2 * NKS; ++j) {
          if constexpr (!kAhead)
            if (j + 1 < 2 * NKS) load_kt(j + 1, (j + 1) & 1);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4 acc = S[j][nb] * gC;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) acc = mma32(kAhead ? Kt[j][pp] : kt[j & 1][pp], Wtb[pp][nb], acc);
            S[j][nb] = acc;
          }
        }
        // outputs of the whole slice from the staging: each lane stores 2 NB
        // runs of 8 value columns of one token; wave c covers 64 / NCW tokens
        constexpr int TW = CH / NCW;
#pragma unroll
        for (int k = 0; k < 2 * NB; ++k) {
          const int q = 16 * (g + 4 * k);
          const int tb = TW * wave + q % TW, cgp = q / TW;  // token base, 8-column group
          const bf16* src = sO + (8 * cgp + (l16 >> 2)) * SO + tb + 4 * (l16 & 3);
          const bf16x8 v = cat8(lds_tr4(src), lds_tr4(src + 4 * SO));
          const int t = n * CH + tb + l16;
          if (t < T) *reinterpret_cast<bf16x8*>(og + t * H * DV + 8 * cgp) = v;
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
    // All four producer waves write the k rows of chunk n and the gated v
    // rows of chunk n - 1 to LDS (phase 1: the consumers read Z of chunk
    // n - 1 in phase 2 of this step) and compute the Gram tiles (phase 2);
    // waves 0 and 1 then compute A = (I + T)^-1 (phase 3), splitting its last
    // level, while waves 2 and 3 write the q rows of chunk n + 1 (phase 3: the
    // consumers read q in phase 1 only, so the buffer of the chunk that they
    // apply is free by then) and load those of chunk n + 2.  Waves 2 and 3
    // share their SIMDs with the consumers and bound phase 1, so they issue
    // their k and v loads behind their Gram tiles instead.
    // One loop per producer wave, with the wave's role fixed at compile time:
    // a single loop with run-time role branches makes the register allocator
    // move prefetched registers at the branch joins, which waits for loads
    // still in flight.
    auto producer = [&](auto pwc) {
    constexpr int pw = decltype(pwc)::value;
    // the chunk scalars (prefix sum of the log-decay) come from wave 1, which
    // has a SIMD of its own (with two consumer waves, producer waves 2 and 3
    // share their SIMDs with them)
    constexpr int kScanWave = 1;
    constexpr bool kRowWave = pw >= 2;  // writes the q rows
    constexpr bool kRecWave = PRE && pw < 2;  // record mode: copies the record
    const int pt = tid - 64 * NCW;
    constexpr int CG = DK / 8, TG = 256 / CG, TPT = CH / TG;      // k: 8 channels x TPT tokens
    constexpr int QTG = 128 / CG, QPT = CH / QTG;                 // q: over waves 2, 3
    constexpr int VG = DVS / 8, VTG = 256 / VG, VPT = (CH + VTG - 1) / VTG;  // v: 8 columns x VPT tokens
    const int c0 = (pt % CG) * 8, tk0 = (pt / CG) * TPT;
    const int rt = pt - 128;  // lane index over waves 2 and 3
    const int qc0 = (rt % CG) * 8, tq0 = (rt / CG) * QPT;
    const int vv0 = (pt % VG) * 8, vtq0 = (pt / VG) * VPT;
    const bool vact = vtq0 < CH;  // wave-uniform
    const bf16* qg = reinterpret_cast<const bf16*>(p.q) + seq0 * DK;
    const bf16* kg = reinterpret_cast<const bf16*>(p.k) + seq0 * DK;
    const bf16* vg = reinterpret_cast<const bf16*>(p.v) + seq0 * DV + vbase;
    const bool has_decay = p.decay != 0;
    // with no decay the log-decay is read from a stand-in buffer of at least
    // B*T*H floats (q) and discarded
    const float* gsrc = has_decay ? p.g + seq0 : reinterpret_cast<const float*>(p.q) + seq0;
    const float* beta_seq = p.beta + seq0;
    const float* w_seq = write_ch ? p.w + seq0 * DV + vbase : nullptr;

    // inputs of coming chunks, prefetched into registers.  Loads are
    // unconditional, at token indices clamped to T - 1; rows past the end are
    // zeroed when they are written to LDS.
    struct Raw {
      bf16x8 k[TPT];
      float gs, bs;  // scan wave: log-decay and beta of token t0 + lane
      bf16x8 q[kRowWave ? QPT : 1];
      bf16x8 v[VPT];
      f32x4 w[write_ch ? VPT : 1][2];
      float vb[write_ch ? 1 : VPT];  // beta of the v rows (the beta write gate)
      u32x4 rc[kRecWave ? 6 : 1];    // record mode: this lane's pieces of the chunk's record
    };
    // Loads address the chunk from a uniform base with 32-bit per-lane byte
    // offsets (row of the token within the chunk), so that they take the
    // scalar-base form and keep no 64-bit addresses in vector registers.
    auto ldg = [&](auto vt, const void* base, unsigned byteoff) __attribute__((always_inline)) {
      using V = decltype(vt);
      return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byteoff);
    };
    // token row (t * H) of token t of chunk n relative to the chunk start
    auto row = [&](int n, int t) __attribute__((always_inline)) -> unsigned {
      return (unsigned)(min(n * CH + t, T - 1) - n * CH) * H;
    };
    auto load_k = [&](int n, Raw& R) {
      const bf16* kc = kg + (size_t)n * CH * H * DK;
#pragma unroll
      for (int u = 0; u < TPT; ++u) R.k[u] = ldg(bf16x8{}, kc, 2 * (row(n, tk0 + u) * DK + c0));
    };
    auto load_gb = [&](int n, Raw& R) {
      const unsigned r = row(n, lane);
      R.gs = ldg(float{}, gsrc + (size_t)n * CH * H, 4 * r);
      R.bs = ldg(float{}, beta_seq + (size_t)n * CH * H, 4 * r);
    };
    auto load_q = [&](int n, Raw& R) {
      const bf16* qc = qg + (size_t)n * CH * H * DK;
#pragma unroll
      for (int u = 0; u < QPT; ++u) R.q[u] = ldg(bf16x8{}, qc, 2 * (row(n, tq0 + u) * DK + qc0));
    };
    auto load_v = [&](int n, Raw& R) {
      if (!vact) return;
      const bf16* vc = vg + (size_t)n * CH * H * DV;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const unsigned r = row(n, vtq0 + u);
        R.v[u] = ldg(bf16x8{}, vc, 2 * (r * DV + vv0));
        if constexpr (!write_ch) R.vb[u] = ldg(float{}, beta_seq + (size_t)n * CH * H, 4 * r);
      }
    };
    // per-channel write gate: loaded one phase before its use rather than a
    // step before, so that its registers are not live during the Gram tiles
    auto load_w = [&](int n, Raw& R) {
      if (!vact) return;
      const float* wc = w_seq + (size_t)n * CH * H * DV;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const unsigned o = row(n, vtq0 + u) * DV + vv0;
        R.w[u][0] = ldg(f32x4{}, wc, 4 * o);
        R.w[u][1] = ldg(f32x4{}, wc, 4 * o + 16);
      }
    };

    // PRE: pieces 0-319 of a record are the A triangle, 320-639 the A_qk
    // triangle, 640-723 the scalars; waves 0 and 1 copy them, waves 2 and 3
    // write the q rows.  Lane pt < 128: pieces pt and pt + 128 of each
    // triangle; the last 64 pieces of A go to wave 0, those of A_qk to wave
    // 1; scalar pieces 0-63 to wave 0, 64-83 to wave 1.
    static_assert(PipeRec::NPIECE == 2 * PipeRec::PIECES_A + NSC / 4 && NSC / 4 > 64 && NSC / 4 <= 128,
                  "record pieces");
    constexpr int qAqk = PipeRec::oAqk / 16, qSc = PipeRec::oSc / 16;
    const int px = pt & 63;
    const int rxq = pw == 0 ? 256 + px : qAqk + 256 + px;           // extra triangle piece
    const int rsq = qSc + (pw == 0 ? px : 64 + min(px, NSC / 4 - 65));  // scalar piece
    auto load_rec = [&](int n, Raw& R) __attribute__((always_inline)) {
      if constexpr (kRecWave) {
        const u32x4* r0 = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.ws) +
                                                         ((size_t)bh * nchunks + n) * PipeRec::BYTES);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          R.rc[k] = r0[pt + 128 * k];
          R.rc[2 + k] = r0[qAqk + pt + 128 * k];
        }
        R.rc[4] = r0[rxq];
        R.rc[5] = r0[rsq];
      }
    };
    auto write_rec = [&](int buf, const Raw& R) __attribute__((always_inline)) {
      if constexpr (kRecWave) {
        bf16* A = sAcm + buf * CH * SC;
        bf16* Aq = sAqk + buf * CH * SC;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const TriPiece a = tri_upper_piece(pt + 128 * k), b = tri_lower_piece(pt + 128 * k);
          *reinterpret_cast<u32x4*>(A + a.row * SC + a.col * 8) = R.rc[k];
          *reinterpret_cast<u32x4*>(Aq + b.row * SC + b.col * 8) = R.rc[2 + k];
        }
        const TriPiece x = pw == 0 ? tri_upper_piece(256 + px) : tri_lower_piece(256 + px);
        *reinterpret_cast<u32x4*>((pw == 0 ? A : Aq) + x.row * SC + x.col * 8) = R.rc[4];
        if (pw == 0 || px < NSC / 4 - 64) *reinterpret_cast<u32x4*>(sSc + buf * NSC + 4 * (rsq - qSc)) = R.rc[5];
      }
    };
    // PRE, phase 3: K^T of chunk n (channel-major runs of 8 tokens) from its
    // k rows, for the consumers' b128 fragment reads.  Lane pt, k: 16-lane
    // group 4 (pt / 64) + g + 16 k takes channels 16 (group / 8) + l16, run
    // group % 8 (two transposing reads of 4 tokens x 16 channels).
    auto rows_kt = [&](int buf) __attribute__((always_inline)) {
      const bf16* Kb = sK + buf * CH * SK;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int grp = 4 * pw + g + 16 * k, r = grp & 7, cb = 16 * (grp >> 3);
        const bf16* src = Kb + (8 * r + (l16 >> 2)) * SK + cb + 4 * (l16 & 3);
        const bf16x8 v = cat8(lds_tr4(src), lds_tr4(src + 4 * SK));
        *reinterpret_cast<bf16x8*>(sKT + kt_off(cb + l16, r)) = v;
      }
    };

    // ---- phase 1: chunk scalars (scan wave), k rows ------------------------
    // (PRE: the scalars come with the record in phase 2, which also takes the
    // q rows of the next chunk: with no Gram tiles or inverse to form, the
    // producers' work of a step fits in the consumers' first two phases)
    auto rows_k = [&](int n, int buf, const Raw& R) {
      const int t0 = n * CH;
      bf16* Kb = sK + buf * CH * SK;
      const bf16x8 zero = {};
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = tk0 + u;
        *reinterpret_cast<bf16x8*>(Kb + t * SK + c0) = (t0 + t < T) ? R.k[u] : zero;
      }
    };
    auto prep = [&](int n, int buf, const Raw& R) {
      const int t0 = n * CH;
      if constexpr (pw == kScanWave) {
        const float G = wave_incl_scan((has_decay && t0 + lane < T) ? R.gs : 0.f);
        float* sc = sSc + buf * NSC;
        const float GC = lane_value(G, 63);
        const float gam = fexp(G);
        sc[L::sG + lane] = G;
        sc[L::sBeta + lane] = R.bs;
        sc[L::sCE + lane] = R.bs * gam;
        sc[L::sGam + lane] = gam;
        sc[L::sTail + lane] = fexp(GC - G);
        if (lane == 0) sc[L::sGC] = fexp(GC);
      }
      rows_k(n, buf, R);
    };
    // ---- phase 3 (waves 2, 3): q rows of chunk n -----------------------------
    auto rows_q = [&](int n, int buf, const Raw& R) {
      const int t0 = n * CH;
      bf16* Qb = sQ + buf * CH * SQ;
      const bf16x8 zero = {};
#pragma unroll
      for (int u = 0; u < QPT; ++u) {
        const int t = tq0 + u;
        *reinterpret_cast<bf16x8*>(Qb + t * SQ + qc0) = (t0 + t < T) ? R.q[u] : zero;
      }
    };
    // ---- phase 1 of the next step: Z = gate * v rows of chunk n --------------
    auto rows_z = [&](int n, int buf, const Raw& R) {
      if (!vact) return;
      const int t0 = n * CH;
      bf16* Zb = sZ;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int t = vtq0 + u;
        const bool ok = t0 + t < T;
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float gate;
          if constexpr (write_ch) gate = e < 4 ? R.w[u][0][e] : R.w[u][1][e - 4];
          else gate = R.vb[u];
          z[e] = ok ? gate * (float)R.v[u][e] : 0.f;
        }
        st8(Zb + t * SZ + vv0, z);
      }
    };
    // ---- phase 2: T and A_qk tiles ------------------------------------------
    // Each producer wave computes both T and A_qk on its (I, J) tiles, so the
    // K_J fragments and the decay factors exp(G_i - G_j) serve both:
    //   wave 0: (3,0) (3,1) (0,0)   wave 1: (2,0) (2,1) (2,2)
    //   wave 2: (1,0) (1,1)         wave 3: (3,2) (3,3)
    // Tiles are computed transposed, D^T = K_J X_I^T, so that each lane holds
    // four consecutive columns j of one row i.  Diagonal blocks of T go to
    // fp32 rows for level 0 of the solve, the others to bf16 rows.
    // (the Q-Delta mix is a template argument: a run-time test inside the
    // k-step loop branches around every fragment)
    auto gram = [&](auto tiles, int buf, auto qm) {
      const float* sc = sSc + buf * NSC;
      scalar_gram_tiles<DK, SK, SQ, SC, TDS, TDB, decltype(qm)::value>(
          tiles, sK + buf * CH * SK, sQ + buf * CH * SQ, sc + L::sG, sc + L::sBeta, lam, sT, sTd,
          sAqk + buf * CH * SC, SC, g, l16);
    };

    // ---- phase 3 (wave 0): A = (I + T)^{-1} ----------------------------------
    // waves 0 and 1 (the scan wave, with a SIMD of its own) split its last level
    auto solve = [&](auto jm, int buf) {
      solve_inverse<SC, TDS, TDB, decltype(jm)::value>(sTd, sT, sAcm + buf * CH * SC, g, l16);
    };

    Raw R;
    if (nchunks > 0) {
      load_k(0, R);
      if constexpr (PRE) load_rec(0, R);
      else if constexpr (pw == kScanWave) load_gb(0, R);
      if constexpr (kRowWave) {
        load_q(0, R);
        rows_q(0, 0, R);
        load_q(min(1, nchunks - 1), R);
      }
    }
    // Prefetches are unconditional, the chunk index clamped to the last one:
    // registers loaded under a condition that the compiler cannot tie to
    // their use stay live across the whole loop.
    for (int n = 0; n < nchunks; ++n) {
      const int buf = n & 1;
      const int nn = min(n + 1, nchunks - 1);
      if constexpr (PRE) rows_k(n, buf, R);
      else prep(n, buf, R);
      if (n > 0) rows_z(n - 1, buf ^ 1, R);
      // (waves 2 and 3 share their SIMDs with the consumers and bound phase
      // 1: their loads go behind their Gram tiles in phase 2)
      if constexpr (PRE || !kRowWave) {
        load_k(nn, R);
        load_v(n, R);
      }
      __syncthreads();
      if constexpr (PRE) {
        // (the consumers have read the q rows of chunk n - 1 in phase 1)
        write_rec(buf, R);
        load_rec(nn, R);
        if constexpr (kRowWave) {
          if (n + 1 < nchunks) rows_q(n + 1, buf ^ 1, R);
          load_q(min(n + 2, nchunks - 1), R);
        }
      } else {
        auto tiles = [&](auto qm) {
          if constexpr (pw == 0) gram(Tiles<3, 3, 0, 3, 1, 0, 0>{}, buf, qm);
          else if constexpr (pw == 1) gram(Tiles<3, 2, 0, 2, 1, 2, 2>{}, buf, qm);
          else if constexpr (pw == 2) gram(Tiles<2, 1, 0, 1, 1>{}, buf, qm);
          else gram(Tiles<2, 3, 2, 3, 3>{}, buf, qm);
        };
        if (qmix) tiles(IC<1>{});
        else tiles(IC<0>{});
        if constexpr (kRowWave) {
          load_k(nn, R);
          load_v(n, R);
        }
        // g and beta are loaded here rather than in phase 3, so that they
        // have arrived when the next step's prefix sum starts
        if constexpr (pw == kScanWave) load_gb(nn, R);
      }
      __syncthreads();
      if constexpr (PRE) {
        // (the consumers have read K^T of chunk n - 1 in phase 2)
        rows_kt(buf);
      } else {
        if constexpr (pw == 0) solve(IC<1>{}, buf);
        if constexpr (pw == kScanWave) solve(IC<2>{}, buf);
        if constexpr (kRowWave) {
          if (n + 1 < nchunks) rows_q(n + 1, buf ^ 1, R);
          load_q(min(n + 2, nchunks - 1), R);
        }
      }
      if constexpr (write_ch) load_w(n, R);
      __syncthreads();
    }
    // Z rows of the last chunk, before the consumers' phase 2 applies it
    if (nchunks > 0) rows_z(nchunks - 1, (nchunks - 1) & 1, R);
    // last step: the consumers apply the last chunk
    __syncthreads();
    __syncthreads();
    __syncthreads();
    };
    switch (wave - NCW) {
      case 0: producer(IC<0>{}); break;
      case 1: producer(IC<1>{}); break;
      case 2: producer(IC<2>{}); break;
      default: producer(IC<3>{}); break;
    }
  }
}

template <int DK, int DVS>
constexpr int pipe_lds_bytes() {
  return PipeLay<DK, DVS>::TOTAL;
}

}  // namespace gdr
