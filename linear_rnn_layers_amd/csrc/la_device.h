// la_device.h -- device building blocks for the gfx950 linear-attention kernels:
// storage conversions, the feature map, MFMA fragments and precision policies,
// and the row staging loop.
//
// MFMA fragment convention (16x16 output tiles, 64-lane wavefront).  For lane
// l let r16 = l % 16 and g = l / 16.  A K=32 contraction step uses
//   A-fragment: 8 values a[e] = A[r16][k(g,e)]         (row r16 of A)
//   B-fragment: 8 values b[e] = B[k(g,e)][r16]         (column r16 of B)
//   accumulator: acc[r] = C[4g + r][r16], r = 0..3
// where k(g,e) is any bijection onto 0..31 used identically by A and B (the
// hardware pairs element e of lane-group g in A with the same slot in B).
// Two maps are used: the standard map k = 8g + e, and the "accumulator map"
// k = 4g + e (e < 4), 16 + 4g + (e - 4) (e >= 4), under which the accumulators
// of two stacked 16x16 tiles are directly a B-fragment of the next product.
// A K=32 step is one v_mfma_f32_16x16x32_bf16, or eight v_mfma_f32_16x16x4_f32
// (step e takes element e of every lane) for float32 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage (upper half of a float32)

constexpr int NT = 256;  // threads per workgroup: four wavefronts
constexpr int CH = 64;   // tokens per chunk: four 16-row blocks, one per wave

struct F8 {
  float v[8];
};

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

// Feature map of "Transformers are RNNs -- part 2/3" eq. 7 with elu's alpha = 1.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }
// Its derivative is 1 for x > 0 and exp(x) otherwise, i.e. min(phi(x), 1).
__device__ __forceinline__ float dphi_from_phi(float p) { return fminf(p, 1.f); }

// ---------------------------------------------------------------- MFMA
enum Pol {
  P_F32 = 0,  // float32 operands: eight 16x16x4 f32 MFMAs per K=32 step
  P_B1 = 1,   // both operands rounded to bf16: one MFMA
  P_B2A = 2,  // A split into bf16 hi + lo, B exact in bf16: two MFMAs
  P_B2B = 3,  // A exact in bf16, B split: two MFMAs
  P_B3 = 4    // both split: hi*hi + hi*lo + lo*hi, three MFMAs
};

__device__ __forceinline__ bf16x8_t cvt8(const F8& x) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x.v[e];
  return r;
}

__device__ __forceinline__ void split8(const F8& x, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = (__bf16)x.v[e];
    hi[e] = h;
    lo[e] = (__bf16)(x.v[e] - (float)h);
  }
}

__device__ __forceinline__ f32x4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int P>
__device__ __forceinline__ void mma(f32x4_t& acc, const F8& a, const F8& b) {
  if constexpr (P == P_F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  } else if constexpr (P == P_B1) {
    acc = mfma_bf16(cvt8(a), cvt8(b), acc);
  } else if constexpr (P == P_B2A) {
    bf16x8_t ah, al;
    split8(a, ah, al);
    bf16x8_t bb = cvt8(b);
    acc = mfma_bf16(al, bb, acc);
    acc = mfma_bf16(ah, bb, acc);
  } else if constexpr (P == P_B2B) {
    bf16x8_t bh, bl;
    split8(b, bh, bl);
    bf16x8_t aa = cvt8(a);
    acc = mfma_bf16(aa, bl, acc);
    acc = mfma_bf16(aa, bh, acc);
  } else {
    bf16x8_t ah, al, bh, bl;
    split8(a, ah, al);
    split8(b, bh, bl);
    acc = mfma_bf16(ah, bl, acc);
    acc = mfma_bf16(al, bh, acc);
    acc = mfma_bf16(ah, bh, acc);
  }
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Accumulators of two stacked tiles as one fragment under the accumulator map.
__device__ __forceinline__ F8 acc2frag(const f32x4_t& a0, const f32x4_t& a1) {
  F8 f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f.v[r] = a0[r];
    f.v[4 + r] = a1[r];
  }
  return f;
}

// ------------------------------------------------------- LDS fragment loads
// 8 consecutive elements (16-byte aligned for float, 16-byte for bf16).
__device__ __forceinline__ F8 ld8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return F8{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}
__device__ __forceinline__ F8 ld8(const bf16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  F8 f;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[2 * i] = __uint_as_float(w[i] << 16);
    f.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return f;
}
__device__ __forceinline__ void ld4(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void ld4(const bf16_t* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(u.x << 16);
  o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16);
  o[3] = __uint_as_float(u.y & 0xffff0000u);
}
// Standard map: row[k0 + 8g + e].
template <typename LT>
__device__ __forceinline__ F8 frag_std(const LT* row, int k0, int g) { return ld8(row + k0 + 8 * g); }
// Accumulator map: row[k0 + 4g + e] (e < 4), row[k0 + 16 + 4g + e - 4] (e >= 4).
template <typename LT>
__device__ __forceinline__ F8 frag_acc(const LT* row, int k0, int g) {
  F8 f;
  ld4(row + k0 + 4 * g, f.v);
  ld4(row + k0 + 16 + 4 * g, f.v + 4);
  return f;
}
// Standard map down a column: base[(k0 + 8g + e) * pitch].
template <typename LT>
__device__ __forceinline__ float lds_get(const LT* p);
template <>
__device__ __forceinline__ float lds_get<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float lds_get<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename LT>
__device__ __forceinline__ F8 frag_col(const LT* col, int pitch, int k0, int g) {
  F8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = lds_get<LT>(col + (k0 + 8 * g + e) * pitch);
  return f;
}

// ----------------------------------------------------------- LDS stores
__device__ __forceinline__ void lds_put(float* p, float x) { *p = x; }
__device__ __forceinline__ void lds_put(bf16_t* p, float x) { *p = f2bf(x); }
__device__ __forceinline__ void lds_put4(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void lds_put4(bf16_t* p, const float* x) {
  uint2 u;
  u.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
  u.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <typename LT, int E>
__device__ __forceinline__ void lds_putE(LT* p, const float* x) {
#pragma unroll
  for (int i = 0; i < E; i += 4) lds_put4(p + i, x + i);
}

// --------------------------------------------------------- global I/O
// E elements per 16-byte vector: 4 floats or 8 bf16.
template <typename T>
struct IO;
template <>
struct IO<float> {
  static constexpr int E = 4;
  __device__ static __forceinline__ void load(const float* p, float* x) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  __device__ static __forceinline__ void store4(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <>
struct IO<bf16_t> {
  static constexpr int E = 8;
  __device__ static __forceinline__ void load(const bf16_t* p, float* x) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void store4(bf16_t* p, const float* x) {
    uint2 u;
    u.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
    u.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

// Visit the CH rows of a [rows, COLS] slab in 16-byte vectors, spread over the
// workgroup.  Rows >= nvalid are presented as zeros with valid = false.  Each
// wavefront covers whole rows with COLS/E consecutive lanes, and every thread
// runs the same number of iterations, so cross-lane reductions inside `f` over
// groups of COLS/E lanes are safe.
template <typename T, int COLS, typename F>
__device__ __forceinline__ void for_rows(const T* base, int nvalid, F&& f) {
  constexpr int E = IO<T>::E;
  constexpr int PR = COLS / E;
  constexpr int TOT = CH * PR;
  static_assert(TOT % NT == 0, "row visit must be uniform over the workgroup");
#pragma unroll
  for (int v = threadIdx.x; v < TOT; v += NT) {
    const int r = v / PR;
    const int c0 = (v % PR) * E;
    float x[E];
    const bool ok = r < nvalid;
    if (ok) {
      IO<T>::load(base + (size_t)r * COLS + c0, x);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
    }
    f(r, c0, x, ok);
  }
}

__device__ __forceinline__ float sum_over_g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
