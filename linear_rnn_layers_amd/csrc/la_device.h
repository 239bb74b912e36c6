// la_device.h -- device building blocks for the gfx950 linear-attention kernels:
// storage conversions, the feature map, bf16 operand planes in LDS, MFMA
// fragments and split-precision products, and the chunk staging helpers.
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
//
// Split precision.  A float32 operand x is staged as NP bf16 "planes"
// x = x0 + x1 (+ x2) + residual, each plane the bf16 rounding of what the
// previous ones leave (residual about 2^-8, 2^-16, 2^-24 of |x| for NP = 1,
// 2, 3).  A product of an NA-plane and an NB-plane operand keeps the terms
// a_i b_j with i + j < max(NA, NB), smallest first, each one
// v_mfma_f32_16x16x32_bf16 with float32 accumulation: (1,1) is a plain bf16
// product, (2,2) is accurate to about 2^-16 with 3 MFMAs, (3,3) to float32
// level with 6 MFMAs -- 2.7x faster than eight v_mfma_f32_16x16x4_f32.
// Operands that are exact in bf16 (bf16 inputs, a 0/1 mask) need one plane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage (upper half of a float32)

constexpr int NT = 256;  // threads per workgroup: four wavefronts

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(bf16_t, h);
}

// Feature map of "Transformers are RNNs -- part 2/3" eq. 7 with elu's alpha = 1.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }
// Its derivative is 1 for x > 0 and exp(x) otherwise, i.e. min(phi(x), 1).
__device__ __forceinline__ float dphi_from_phi(float p) { return fminf(p, 1.f); }

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- splitting
template <int NP>
__device__ __forceinline__ void split(float x, bf16_t* out) {
  float r = x;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const __bf16 h = (__bf16)r;
    out[p] = __builtin_bit_cast(bf16_t, h);
    if (p + 1 < NP) r -= (float)h;
  }
}

template <int N>
struct Frag {
  bf16x8_t p[N];
};

// Fragment of 8 float32 values split into N planes.
template <int N>
__device__ __forceinline__ Frag<N> split8(const float* v) {
  Frag<N> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float r = v[e];
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const __bf16 h = (__bf16)r;
      f.p[p][e] = h;
      if (p + 1 < N) r -= (float)h;
    }
  }
  return f;
}

// Accumulators of two stacked tiles as one fragment under the accumulator map.
template <int N>
__device__ __forceinline__ Frag<N> acc2frag(const f32x4_t& a0, const f32x4_t& a1) {
  const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  return split8<N>(v);
}

// acc += A B keeping the terms a_i b_j, i + j < max(NA, NB), smallest first.
template <int NA, int NB, int FA, int FB>
__device__ __forceinline__ void mmaf(f32x4_t& acc, const Frag<FA>& a, const Frag<FB>& b) {
  static_assert(NA <= FA && NB <= FB, "operand has fewer planes than the product uses");
  constexpr int ORD = NA > NB ? NA : NB;
#pragma unroll
  for (int s = ORD - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i <= s; ++i) {
      const int j = s - i;
      if (i < NA && j < NB) acc = mfma_bf16(a.p[i], b.p[j], acc);
    }
  }
}

// ---------------------------------------------------------- LDS planes
// NP bf16 planes of a ROWS x COLS matrix; every row padded by 8 elements so
// rows are 16-byte aligned and consecutive rows start in different banks.
template <int NP, int ROWS, int COLS>
struct Planes {
  static constexpr int P = COLS + 8;
  bf16_t v[NP][ROWS][P];

  __device__ __forceinline__ void put(int r, int c, float x) {
    bf16_t h[NP];
    split<NP>(x, h);
#pragma unroll
    for (int p = 0; p < NP; ++p) v[p][r][c] = h[p];
  }
  // E consecutive columns (E a multiple of 4) from one row
  template <int E>
  __device__ __forceinline__ void putrow(int r, int c, const float* x) {
#pragma unroll
    for (int i = 0; i < E; i += 4) {
      bf16_t h[4][NP];
#pragma unroll
      for (int q = 0; q < 4; ++q) split<NP>(x[i + q], h[q]);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        uint2 u;
        u.x = (uint32_t)h[0][p] | ((uint32_t)h[1][p] << 16);
        u.y = (uint32_t)h[2][p] | ((uint32_t)h[3][p] << 16);
        *reinterpret_cast<uint2*>(&v[p][r][c + i]) = u;
      }
    }
  }
  // value represented by the planes
  __device__ __forceinline__ float get(int r, int c) const {
    float s = 0.f;
#pragma unroll
    for (int p = NP - 1; p >= 0; --p) s += bf2f(v[p][r][c]);
    return s;
  }
  // four consecutive values of one row
  __device__ __forceinline__ void get4(int r, int c, float* o) const {
    o[0] = o[1] = o[2] = o[3] = 0.f;
#pragma unroll
    for (int p = NP - 1; p >= 0; --p) {
      const uint2 u = *reinterpret_cast<const uint2*>(&v[p][r][c]);
      o[0] += __uint_as_float(u.x << 16);
      o[1] += __uint_as_float(u.x & 0xffff0000u);
      o[2] += __uint_as_float(u.y << 16);
      o[3] += __uint_as_float(u.y & 0xffff0000u);
    }
  }
  // standard map along a row: v[.][row][k0 + 8g + e]
  template <int N>
  __device__ __forceinline__ Frag<N> frag(int row, int k0, int g) const {
    static_assert(N <= NP, "not enough planes");
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p) f.p[p] = *reinterpret_cast<const bf16x8_t*>(&v[p][row][k0 + 8 * g]);
    return f;
  }
  // accumulator map along a row
  template <int N>
  __device__ __forceinline__ Frag<N> frag_acc(int row, int k0, int g) const {
    static_assert(N <= NP, "not enough planes");
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(&v[p][row][k0 + 4 * g]);
      const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(&v[p][row][k0 + 16 + 4 * g]);
      f.p[p] = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return f;
  }
  // standard map down a column: v[.][k0 + 8g + e][col]
  template <int N>
  __device__ __forceinline__ Frag<N> frag_col(int col, int k0, int g) const {
    static_assert(N <= NP, "not enough planes");
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) f.p[p][e] = __builtin_bit_cast(__bf16, v[p][k0 + 8 * g + e][col]);
    return f;
  }
};

// A fragment that is a 0/1 mask (exact in bf16).
__device__ __forceinline__ Frag<1> mask_frag(const bool* on) {
  Frag<1> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.p[0][e] = on[e] ? (__bf16)1.0f : (__bf16)0.0f;
  return f;
}

// --------------------------------------------------------- global I/O
// E elements per 16-byte vector: 4 floats or 8 bf16.
template <typename T>
struct IO;
template <>
struct IO<float> {
  static constexpr int E = 4;
  using raw = float4;
  __device__ static __forceinline__ raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static __forceinline__ void unpack(const raw& a, float* x) {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  __device__ static __forceinline__ void load(const float* p, float* x) { unpack(load_raw(p), x); }
  __device__ static __forceinline__ void store4(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <>
struct IO<bf16_t> {
  static constexpr int E = 8;
  using raw = uint4;
  __device__ static __forceinline__ raw load_raw(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static __forceinline__ void unpack(const raw& u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void load(const bf16_t* p, float* x) { unpack(load_raw(p), x); }
  __device__ static __forceinline__ void store4(bf16_t* p, const float* x) {
    uint2 u;
    u.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
    u.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};

// Register buffer for one chunk (CH rows) of a [rows, COLS] tensor: the
// 16-byte vectors this thread owns.  load() issues the global reads (rows at
// or past `nvalid` are zero); for_each() hands them over for staging.  Each
// wavefront owns whole rows as COLS/E consecutive lanes, so cross-lane
// reductions over groups of COLS/E lanes inside for_each are safe.
template <typename T, int CH, int COLS>
struct RowBuf {
  static constexpr int E = IO<T>::E;
  static constexpr int PR = COLS / E;       // vectors per row
  static constexpr int CNT = CH * PR / NT;  // vectors per thread
  static_assert((CH * PR) % NT == 0, "row visit must be uniform over the workgroup");
  typename IO<T>::raw r[CNT];

  __device__ __forceinline__ void load(const T* base, int nvalid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int v = threadIdx.x + i * NT;
      const int row = v / PR, c0 = (v % PR) * E;
      if (row < nvalid)
        r[i] = IO<T>::load_raw(base + (size_t)row * COLS + c0);
      else
        r[i] = typename IO<T>::raw{};
    }
  }
  template <typename F>
  __device__ __forceinline__ void for_each(int nvalid, F&& f) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int v = threadIdx.x + i * NT;
      const int row = v / PR, c0 = (v % PR) * E;
      float x[E];
      IO<T>::unpack(r[i], x);
      f(row, c0, x, row < nvalid);
    }
  }
};

__device__ __forceinline__ float sum_over_g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
