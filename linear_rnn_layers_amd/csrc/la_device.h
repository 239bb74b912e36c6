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
// Every operand is staged token-major ([token][feature], features contiguous).
// A contraction over features reads fragments along a row (one 16-byte or two
// 8-byte LDS reads per plane); a contraction over tokens reads them down a
// column with the transposing LDS read of gfx950 (ds_read_b64_tr_b16): in
// each group of 16 lanes, lane t receives element t % 4 of the 8-byte rows
// addressed by lanes t / 4 + 4e, e = 0..3.  So if lane a of group g addresses
// row k(g, a / 4) at column n0 + 4 (a % 4), lane t gets X[k(g, e)][n0 + t] --
// a fragment of column n0 + r16 with no transposed copy in LDS.
//
// Split precision.  A float32 operand x is staged as NP bf16 "planes"
// x = x0 + x1 (+ x2) + residual, each plane the bf16 rounding of what the
// previous ones leave (residual about 2^-8, 2^-16, 2^-24 of |x| for NP = 1,
// 2, 3).  A product of an NA-plane and an NB-plane operand keeps the terms
// a_i b_j with i + j < max(NA, NB), smallest first, each one
// v_mfma_f32_16x16x32_bf16 with float32 accumulation: (1,1) is a plain bf16
// product, (2,2) is accurate to about 2^-16 with 3 MFMAs, (3,3) to float32
// level with 6 MFMAs -- 2.7x faster than eight v_mfma_f32_16x16x4_f32.
// Operands that are exact in bf16 (bf16 inputs, 0/1 masks) need one plane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage (upper half of a float32)

constexpr int NT = 256;  // threads per workgroup: four wavefronts

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(bf16_t, h);
}
// two floats rounded to bf16 (nearest even) in one 32-bit word, a in the low half
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float lo2f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi2f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Feature map of "Transformers are RNNs -- part 2/3" eq. 7 with elu's alpha = 1:
// x + 1 for x > 0, exp(x) otherwise, exp taken as 2^(x log2 e) on the
// hardware exponential (relative error about |x| 2^-24 plus one ulp).
__device__ __forceinline__ float phi(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
// Its derivative is 1 for x > 0 and exp(x) otherwise, i.e. min(phi(x), 1).

// Feature-map selection: every kernel takes a flag `fm`; fm = 0 applies eq. 7,
// fm = 1 takes Q and K as feature vectors already (another feature map applied
// by the caller, e.g. polynomial or positive random features): the identity,
// with derivative 1.
__device__ __forceinline__ float feat(float x, int fm) { return fm ? x : phi(x); }
// The derivative from the staged p = feat(x): min(p, 1) for eq. 7, 1 for the
// identity; as one median of three per value (the bound is uniform): the
// median of (p, -inf, 1) is min(p, 1), that of (p, 1, 1) is 1.
__device__ __forceinline__ float dfeat(float p, int fm) {
  return __builtin_amdgcn_fmed3f(p, fm ? 1.f : -__builtin_inff(), 1.f);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4_t mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- splitting
// NP planes of 2W consecutive floats, each plane packed in W 32-bit words.
template <int NP, int W>
__device__ __forceinline__ void split_pk(const float* x, uint32_t (*out)[W]) {
  float r[2 * W];
#pragma unroll
  for (int e = 0; e < 2 * W; ++e) r[e] = x[e];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t w = pk2(r[2 * i], r[2 * i + 1]);
      out[p][i] = w;
      if (p + 1 < NP) {
        r[2 * i] -= lo2f(w);
        r[2 * i + 1] -= hi2f(w);
      }
    }
  }
}

template <int N>
struct Frag {
  bf16x8_t p[N];
};

// Fragment of 8 float32 values split into N planes.
template <int N>
__device__ __forceinline__ Frag<N> split8(const float* v) {
  uint32_t u[N][4];
  split_pk<N, 4>(v, u);
  Frag<N> f;
#pragma unroll
  for (int p = 0; p < N; ++p) f.p[p] = __builtin_bit_cast(bf16x8_t, make_uint4(u[p][0], u[p][1], u[p][2], u[p][3]));
  return f;
}

// Accumulators of two stacked tiles as one fragment under the accumulator map.
template <int N>
__device__ __forceinline__ Frag<N> acc2frag(const f32x4_t& a0, const f32x4_t& a1) {
  const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  return split8<N>(v);
}

// The all-ones fragment (exact in bf16): as an A operand it sums a B operand
// over k into every row of the tile; as a B operand, into every column.
__device__ __forceinline__ Frag<1> ones_frag() {
  Frag<1> f;
  const __bf16 one = (__bf16)1.0f;
  f.p[0] = bf16x8_t{one, one, one, one, one, one, one, one};
  return f;
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

// The same product for NTL tiles at once, acc[t] += A[t] B (one B) or
// acc[t] += A B[t] (one A), issued term by term across the tiles: consecutive
// MFMAs then write different accumulators, so the matrix core does not wait
// for one tile's result before the next instruction (a product of one tile
// alone is a chain of dependent accumulations).
template <int NA, int NB, int NTL, int FA, int FB>
__device__ __forceinline__ void mmaf_tiles(f32x4_t (&acc)[NTL], const Frag<FA> (&a)[NTL], const Frag<FB>& b) {
  static_assert(NA <= FA && NB <= FB, "operand has fewer planes than the product uses");
  constexpr int ORD = NA > NB ? NA : NB;
#pragma unroll
  for (int s = ORD - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i <= s; ++i) {
      const int j = s - i;
      if (i < NA && j < NB) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) acc[t] = mfma_bf16(a[t].p[i], b.p[j], acc[t]);
      }
    }
  }
}
template <int NA, int NB, int NTL, int FA, int FB>
__device__ __forceinline__ void mmaf_tiles(f32x4_t (&acc)[NTL], const Frag<FA>& a, const Frag<FB> (&b)[NTL]) {
  static_assert(NA <= FA && NB <= FB, "operand has fewer planes than the product uses");
  constexpr int ORD = NA > NB ? NA : NB;
#pragma unroll
  for (int s = ORD - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i <= s; ++i) {
      const int j = s - i;
      if (i < NA && j < NB) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) acc[t] = mfma_bf16(a.p[i], b[t].p[j], acc[t]);
      }
    }
  }
}

template <int NA, int NB, int NTL, int FA, int FB>
__device__ __forceinline__ void mmaf_tiles(f32x4_t (&acc)[NTL], const Frag<FA> (&a)[NTL], const Frag<FB> (&b)[NTL]) {
  static_assert(NA <= FA && NB <= FB, "operand has fewer planes than the product uses");
  constexpr int ORD = NA > NB ? NA : NB;
#pragma unroll
  for (int s = ORD - 1; s >= 0; --s) {
#pragma unroll
    for (int i = 0; i <= s; ++i) {
      const int j = s - i;
      if (i < NA && j < NB) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) acc[t] = mfma_bf16(a[t].p[i], b[t].p[j], acc[t]);
      }
    }
  }
}

// ------------------------------------------------------ transposed read
__device__ __forceinline__ bf16x4_t lds_read_tr4(const bf16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4_t, r);
}

__device__ __forceinline__ bf16x8_t cat44(const bf16x4_t& lo, const bf16x4_t& hi) {
  return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------- LDS planes
// NP bf16 planes of a ROWS x COLS row-major matrix; rows padded by PAD
// elements (rows stay 16-byte aligned and consecutive rows start in
// different banks).
template <int NP, int ROWS, int COLS, int PAD = 8>
struct Planes {
  static constexpr int P = COLS + PAD;
  static_assert(P % 8 == 0, "rows must stay 16-byte aligned");
  alignas(16) bf16_t v[NP][ROWS][P];

  // 8 (or 4) consecutive values of one row, split into the planes
  __device__ __forceinline__ void put8(int r, int c, const float* x) {
    uint32_t u[NP][4];
    split_pk<NP, 4>(x, u);
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<uint4*>(&v[p][r][c]) = make_uint4(u[p][0], u[p][1], u[p][2], u[p][3]);
  }
  __device__ __forceinline__ void put4(int r, int c, const float* x) {
    uint32_t u[NP][2];
    split_pk<NP, 2>(x, u);
#pragma unroll
    for (int p = 0; p < NP; ++p) *reinterpret_cast<uint2*>(&v[p][r][c]) = make_uint2(u[p][0], u[p][1]);
  }
  template <int E>
  __device__ __forceinline__ void put(int r, int c, const float* x) {
    static_assert(E == 4 || E == 8, "4 or 8 values");
    if constexpr (E == 8)
      put8(r, c, x);
    else
      put4(r, c, x);
  }
  // one value (all planes)
  __device__ __forceinline__ void put1(int r, int c, float x) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const __bf16 h = (__bf16)x;
      v[p][r][c] = __builtin_bit_cast(bf16_t, h);
      if (p + 1 < NP) x -= (float)h;
    }
  }
  // four consecutive values of one row (sum of the planes, smallest first)
  __device__ __forceinline__ void get4(int r, int c, float* o) const {
#pragma unroll
    for (int p = NP - 1; p >= 0; --p) {
      const uint2 u = *reinterpret_cast<const uint2*>(&v[p][r][c]);
      const float x[4] = {lo2f(u.x), hi2f(u.x), lo2f(u.y), hi2f(u.y)};
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = p == NP - 1 ? x[q] : o[q] + x[q];
    }
  }
  // row fragment, standard map: v[.][row][k0 + 8g + e]
  template <int N>
  __device__ __forceinline__ Frag<N> frag(int row, int k0, int g) const {
    static_assert(N <= NP, "not enough planes");
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p) f.p[p] = *reinterpret_cast<const bf16x8_t*>(&v[p][row][k0 + 8 * g]);
    return f;
  }
  // column fragment, standard map: v[.][k0 + 8g + e][n0 + r16]  (a = r16)
  template <int N>
  __device__ __forceinline__ Frag<N> tfrag(int k0, int n0, int g, int a) const {
    static_assert(N <= NP, "not enough planes");
    const int r = k0 + 8 * g + (a >> 2), c = n0 + 4 * (a & 3);
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p) f.p[p] = cat44(lds_read_tr4(&v[p][r][c]), lds_read_tr4(&v[p][r + 4][c]));
    return f;
  }
  // column fragment, accumulator map
  template <int N>
  __device__ __forceinline__ Frag<N> tfrag_acc(int k0, int n0, int g, int a) const {
    static_assert(N <= NP, "not enough planes");
    const int r = k0 + 4 * g + (a >> 2), c = n0 + 4 * (a & 3);
    Frag<N> f;
#pragma unroll
    for (int p = 0; p < N; ++p) f.p[p] = cat44(lds_read_tr4(&v[p][r][c]), lds_read_tr4(&v[p][r + 16][c]));
    return f;
  }
  // zero columns [c0, c1) of every row and plane (cooperative: nth threads)
  __device__ __forceinline__ void zero_cols(int c0, int c1, int nth = NT) {
    const int w = c1 - c0;
    for (int i = threadIdx.x; i < NP * ROWS * w; i += nth) {
      const int p = i / (ROWS * w), rem = i % (ROWS * w);
      v[p][rem / w][c0 + rem % w] = 0;
    }
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
  __device__ static __forceinline__ void store4(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  __device__ static __forceinline__ void load4(const float* p, float* x) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  // four consecutive elements as loaded (kept in flight), then widened
  using raw4 = float4;
  __device__ static __forceinline__ raw4 load_raw4(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static __forceinline__ raw4 zero_raw4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static __forceinline__ void unpack4(const raw4& a, float* x) {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
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
      x[2 * i] = lo2f(w[i]);
      x[2 * i + 1] = hi2f(w[i]);
    }
  }
  __device__ static __forceinline__ void store4(bf16_t* p, const float* x) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pk2(x[0], x[1]), pk2(x[2], x[3]));
  }
  __device__ static __forceinline__ void load4(const bf16_t* p, float* x) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = lo2f(u.x); x[1] = hi2f(u.x); x[2] = lo2f(u.y); x[3] = hi2f(u.y);
  }
  using raw4 = uint2;
  __device__ static __forceinline__ raw4 load_raw4(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static __forceinline__ raw4 zero_raw4() { return make_uint2(0u, 0u); }
  __device__ static __forceinline__ void unpack4(const raw4& u, float* x) {
    x[0] = lo2f(u.x); x[1] = hi2f(u.x); x[2] = lo2f(u.y); x[3] = hi2f(u.y);
  }
};

// Register buffer for one chunk (CH rows) of a [rows, COLS] tensor: the
// 16-byte vectors this thread owns.  load() issues the global reads (rows at
// or past `nvalid` are zero); the stage_* calls write them to LDS planes.
// Each wavefront owns whole rows as COLS/E consecutive lanes, so cross-lane
// reductions over groups of COLS/E lanes are safe.  A full chunk is read
// from a uniform base plus this thread's fixed 32-bit byte offsets, with no
// per-row test; only a partial chunk takes the masked path.
// When a chunk has fewer vectors than the workgroup has threads, the
// threads [OFF, OFF + VEC) -- whole wavefronts -- hold them, so that several
// tensors can be spread over different wavefronts.
template <typename T, int CH, int COLS, int NTH = NT, int OFF = 0>
struct RowBuf {
  static constexpr int E = IO<T>::E;
  static constexpr int PR = COLS / E;                  // vectors per row
  static constexpr int VEC = CH * PR;                  // vectors per chunk
  static constexpr int VT = VEC < NTH ? VEC : NTH;     // threads holding vectors
  static constexpr int CNT = VEC / VT;                 // vectors per thread
  static_assert(VEC % VT == 0 && VT % 64 == 0 && OFF % 64 == 0 && OFF + VT <= NTH,
                "row visit must be uniform over each wavefront");
  typename IO<T>::raw r[CNT];

  __device__ static __forceinline__ int te() { return (int)threadIdx.x - OFF; }
  __device__ static __forceinline__ bool owns() { return VEC >= NTH || (te() >= 0 && te() < VT); }
  __device__ static __forceinline__ int row_of(int i) { return (te() + i * VT) / PR; }
  __device__ static __forceinline__ int col_of(int i) { return ((te() + i * VT) % PR) * E; }
  __device__ static __forceinline__ uint32_t byte_off(int i) {
    return (uint32_t)(row_of(i) * COLS + col_of(i)) * (uint32_t)sizeof(T);
  }

  __device__ __forceinline__ void load(const T* base, int nvalid) {
    if (!owns()) return;
    const char* b = reinterpret_cast<const char*>(base);
    if (nvalid >= CH) {
#pragma unroll
      for (int i = 0; i < CNT; ++i) r[i] = *reinterpret_cast<const typename IO<T>::raw*>(b + byte_off(i));
    } else {
#pragma unroll
      for (int i = 0; i < CNT; ++i) {
        if (row_of(i) < nvalid)
          r[i] = *reinterpret_cast<const typename IO<T>::raw*>(b + byte_off(i));
        else
          r[i] = typename IO<T>::raw{};
      }
    }
  }
  // Stage values that are exact in bf16 into a one-plane matrix: bf16 input
  // is copied as it is; float32 input is split into the planes.  (Rows past
  // the end were loaded as zeros.)
  template <int NP, int ROWS, int PC, int PAD>
  __device__ __forceinline__ void stage_values(Planes<NP, ROWS, PC, PAD>& dst) const {
    if (!owns()) return;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int row = row_of(i), c0 = col_of(i);
      if constexpr (sizeof(T) == 2 && NP == 1) {
        *reinterpret_cast<uint4*>(&dst.v[0][row][c0]) = r[i];
      } else {
        float x[E];
        IO<T>::unpack(r[i], x);
        dst.template put<E>(row, c0, x);
      }
    }
  }
  // Stage phi of the values (rows past `nvalid` are zero), optionally also
  // as float32 into a [CH][F32C] array.
  template <int NP, int ROWS, int PC, int PAD, int F32C = 0>
  __device__ __forceinline__ void stage_phi(Planes<NP, ROWS, PC, PAD>& dst, int nvalid, float* f32 = nullptr,
                                            int fm = 0) const {
    if (!owns()) return;
    const bool full = nvalid >= CH;
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int row = row_of(i), c0 = col_of(i);
      float x[E];
      IO<T>::unpack(r[i], x);
      if (full) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = feat(x[e], fm);
      } else {
        const bool ok = row < nvalid;
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = ok ? feat(x[e], fm) : 0.f;
      }
      dst.template put<E>(row, c0, x);
      if constexpr (F32C > 0) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
          *reinterpret_cast<float4*>(f32 + row * F32C + c0 + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
      }
    }
  }
};

__device__ __forceinline__ float sum_over_g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
