// Shared device helpers for the gfx950 kernels: vector types, MFMA tile
// products over LDS views, fragment loads and accumulator stores.
//
// MFMA lane layouts used throughout (16x16 output tiles, wave64):
//   v_mfma_f32_16x16x32_bf16: A/B fragment of lane l = 8 consecutive k values
//       (k = 8*(l>>4) .. +7) of row/column (l & 15).
//   v_mfma_f32_16x16x4_f32:   A/B fragment of lane l = 1 value, k = l>>4.
//   accumulator (both):       lane l holds D[4*(l>>4) + r][l & 15], r = 0..3.
// A tile product D = X * Y therefore reads X with k contiguous (row-major X)
// and Y^T with k contiguous, and its accumulator stores 4 consecutive rows of
// one column, i.e. a contiguous vector of D^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4, 8 within each 16-lane row, then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ float wave_incl_scan(float x) {
#define GDR_DPP_ADD(ctrl, rmask)                                                                    \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rmask, \
                                                              0xf, false))
  GDR_DPP_ADD(0x111, 0xf);  // row_shr:1
  GDR_DPP_ADD(0x112, 0xf);  // row_shr:2
  GDR_DPP_ADD(0x114, 0xf);  // row_shr:4
  GDR_DPP_ADD(0x118, 0xf);  // row_shr:8
  GDR_DPP_ADD(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  GDR_DPP_ADD(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef GDR_DPP_ADD
  return x;
}

// an integer as a type (compile-time roles and levels of lambdas)
template <int N>
struct IC {
  static constexpr int value = N;
};

// sum over the lanes of a wave (every lane gets the total)
__device__ __forceinline__ float wave_sum(float s) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
  return s;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// sum over the 64 lanes of a wave as the last lane of its DPP prefix sum
// (every lane active; the result is wave-uniform)
__device__ __forceinline__ float wave_total(float x) { return lane_value(wave_incl_scan(x), 63); }

// 4 x 4 transpose across the lanes of a quad: lane j of the quad holds row j
// of a block in x; afterwards it holds column j.  Two exchanges, with the
// partners j ^ 1 and j ^ 2 (DPP quad permutations); element k is taken from
// the partner where bit 0 (first exchange) or bit 1 (second) of k ^ j is set.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int j) {
  auto from = [](float v, auto ctrl) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                              0xf, 0xf, true));
  };
  f32x4 y;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float o = from(x[k ^ 1], IC<0xB1>{});
    y[k] = ((k ^ j) & 1) ? o : x[k];
  }
  f32x4 z;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float o = from(y[k ^ 2], IC<0x4E>{});
    z[k] = ((k ^ j) & 2) ? o : y[k];
  }
  return z;
}

// A matrix in LDS: element (r, c) at p[r * rs + c * cs].
template <class T>
struct View {
  T* p;
  int rs, cs;
};

template <class T>
__device__ __forceinline__ View<T> view(T* p, int rs, int cs) {
  return View<T>{p, rs, cs};
}

// ---- MFMA traits ---------------------------------------------------------
template <class T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KS = 32;
  typedef bf16x8 frag;
  // rows r0..r0+15, k in [k0, k0+32).  The view must have cs == 1.
  __device__ static __forceinline__ frag load(View<bf16> v, int r0, int k0, int lane) {
    return *reinterpret_cast<const frag*>(v.p + (r0 + (lane & 15)) * v.rs + k0 + ((lane >> 4) << 3));
  }
  // as load(), with zeros for k >= klim (klim - k0 a multiple of 8); branch-free
  __device__ static __forceinline__ frag loadm(View<bf16> v, int r0, int k0, int klim, int lane) {
    const frag f = load(v, r0, k0, lane);
    const frag z = {};
    return (k0 + ((lane >> 4) << 3) < klim) ? f : z;
  }
  __device__ static __forceinline__ f32x4 mma(f32x4 c, frag a, frag b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  typedef float frag;
  __device__ static __forceinline__ frag load(View<float> v, int r0, int k0, int lane) {
    return v.p[(r0 + (lane & 15)) * v.rs + (k0 + (lane >> 4)) * v.cs];
  }
  __device__ static __forceinline__ frag loadm(View<float> v, int r0, int k0, int klim, int lane) {
    const float f = load(v, r0, k0, lane);
    return (k0 + (lane >> 4) < klim) ? f : 0.f;
  }
  __device__ static __forceinline__ f32x4 mma(f32x4 c, frag a, frag b) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// acc += A[i0:i0+16, ak0:ak0+K] * B[bk0:bk0+K, j0:j0+16], with B given as its
// transpose BT (BT[j][k] = B[k][j]).  K is a compile-time multiple of the
// MFMA k-step; all fragments are loaded before the MFMA chain.
template <int K, class T>
__device__ __forceinline__ f32x4 tmm(f32x4 acc, View<T> A, int i0, int ak0, View<T> BT, int j0, int bk0,
                                     int lane) {
  constexpr int KS = Mma<T>::KS, NK = K / KS;
  static_assert(K % KS == 0, "K must be a multiple of the k-step");
  typename Mma<T>::frag a[NK], b[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    a[s] = Mma<T>::load(A, i0, ak0 + s * KS, lane);
    b[s] = Mma<T>::load(BT, j0, bk0 + s * KS, lane);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = Mma<T>::mma(acc, a[s], b[s]);
  return acc;
}

// As tmm over an exact range of K16 (a multiple of 16) k values, masking the
// lanes past the range in the last k-step.
template <int K16, class T>
__device__ __forceinline__ f32x4 tmm_exact(f32x4 acc, View<T> A, int i0, int ak0, View<T> BT, int j0,
                                           int bk0, int lane) {
  constexpr int KS = Mma<T>::KS, NK = (K16 + KS - 1) / KS;
  typename Mma<T>::frag a[NK], b[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    a[s] = Mma<T>::loadm(A, i0, ak0 + s * KS, ak0 + K16, lane);
    b[s] = Mma<T>::loadm(BT, j0, bk0 + s * KS, bk0 + K16, lane);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) acc = Mma<T>::mma(acc, a[s], b[s]);
  return acc;
}

// Store an accumulator tile into out(i, j) for i = i0 + 4*(lane>>4) + r,
// j = j0 + (lane & 15).  tst_vec requires out.rs == 1 (the four rows of one
// lane are contiguous); tst_sca works for any strides.
__device__ __forceinline__ void tst_vec(View<bf16> out, int i0, int j0, f32x4 d, int lane) {
  const int i = i0 + ((lane >> 4) << 2), j = j0 + (lane & 15);
  *reinterpret_cast<bf16x4*>(out.p + i + j * out.cs) = __builtin_convertvector(d, bf16x4);
}
__device__ __forceinline__ void tst_vec(View<float> out, int i0, int j0, f32x4 d, int lane) {
  const int i = i0 + ((lane >> 4) << 2), j = j0 + (lane & 15);
  *reinterpret_cast<f32x4*>(out.p + i + j * out.cs) = d;
}
template <class T>
__device__ __forceinline__ void tst_sca(View<T> out, int i0, int j0, f32x4 d, int lane) {
  const int i = i0 + ((lane >> 4) << 2), j = j0 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) out.p[(i + r) * out.rs + j * out.cs] = (T)d[r];
}

// ---- 8-wide vectors for global loads and LDS stores ----------------------
template <class T>
struct V8;
template <>
struct V8<bf16> {
  bf16x8 x;
  __device__ __forceinline__ float operator[](int i) const { return (float)x[i]; }
};
template <>
struct V8<float> {
  f32x4 a, b;
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

__device__ __forceinline__ V8<bf16> ld8(const bf16* p) {
  return V8<bf16>{*reinterpret_cast<const bf16x8*>(p)};
}
__device__ __forceinline__ V8<float> ld8(const float* p) {
  return V8<float>{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
}
template <class T>
__device__ __forceinline__ V8<T> zero8() {
  V8<T> z;
  if constexpr (sizeof(T) == 2) {
    z.x = bf16x8{};
  } else {
    z.a = f32x4{};
    z.b = f32x4{};
  }
  return z;
}
template <class T>
__device__ __forceinline__ V8<T> sel8(bool keep, V8<T> v) {
  return keep ? v : zero8<T>();
}

// 8 floats -> 8 elements of T at p (16-byte aligned for bf16, 32 for fp32)
__device__ __forceinline__ void st8(bf16* p, const float* f) {
  f32x4 a = {f[0], f[1], f[2], f[3]}, b = {f[4], f[5], f[6], f[7]};
  bf16x4 x = __builtin_convertvector(a, bf16x4), y = __builtin_convertvector(b, bf16x4);
  bf16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  *reinterpret_cast<bf16x8*>(p) = z;
}
__device__ __forceinline__ void st8(float* p, const float* f) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// N consecutive elements (N = 1, 2, 4) from floats
template <int N>
__device__ __forceinline__ void stn(bf16* p, const float* f) {
  if constexpr (N == 4) {
    *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector((f32x4{f[0], f[1], f[2], f[3]}), bf16x4);
  } else if constexpr (N == 2) {
    *reinterpret_cast<bf16x2*>(p) = __builtin_convertvector((f32x2{f[0], f[1]}), bf16x2);
  } else {
    p[0] = (bf16)f[0];
  }
}
template <int N>
__device__ __forceinline__ void stn(float* p, const float* f) {
  if constexpr (N == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  } else if constexpr (N == 2) {
    *reinterpret_cast<f32x2*>(p) = f32x2{f[0], f[1]};
  } else {
    p[0] = f[0];
  }
}

// store 4 consecutive outputs to global memory
__device__ __forceinline__ void gst4(bf16* p, f32x4 d) {
  *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector(d, bf16x4);
}
__device__ __forceinline__ void gst4(float* p, f32x4 d) { *reinterpret_cast<f32x4*>(p) = d; }

}  // namespace gdr
