// la_feature.h -- gfx950 kernels for feature maps other than elu + 1, whose
// output feeds the attention kernels in feature mode (fm = 1).
//
// "Linear Attention/zh", feature maps: positive random features (Performer,
// phi(x) proportional to exp(W x - |x|^2 / 2)) and the truncated polynomial
// map phi(x) = (1, x, x (x) x); "Transformers are RNNs -- part 2/3", section
// 3.2.1: the degree-2 polynomial kernel has an exact feature map of size
// about D^2.
//
// Random features: phi(x)_c = exp(w_c . x - |x|^2 / 2) / sqrt(C) with a
// caller-supplied projection W [H, C, Din] (float32).  The projection W x of
// a 64-token chunk is a dense contraction over Din, done as 16x16 MFMA tiles
// on bf16 planes (la_device.h): wave w owns tokens 16w..16w+15, the tile
// output is [feature][token], so each lane stores four consecutive features
// of one token.  The vector-Jacobian product dX = sum_c dPhi_c phi_c (w_c -
// x) recomputes phi in float32, forms G = dPhi * phi in registers and
// contracts it with W over the features, the accumulators serving directly
// as the next product's operand (accumulator map).
//
// Polynomial features: one thread per token writes (1, x, x_a x_b, 0...).
#pragma once

#include "la_kernels.h"

namespace la {

// Planes of X and W: float32 storage keeps float32 level (the exponent
// amplifies an absolute error of w . x into a relative one); bf16 inputs are
// exact in one plane and W takes two.
template <typename T>
struct FPrec;
template <>
struct FPrec<bf16_t> {
  static constexpr int X = 1, W = 2, G = 2;
};
template <>
struct FPrec<float> {
  static constexpr int X = 3, W = 3, G = 3;
};

// W of one head into planes [C][DIN] (cooperative).
template <int NP, int C, int DIN>
__device__ __forceinline__ void stage_w(Planes<NP, C, DIN>& wt, const float* w) {
  for (int i = 4 * threadIdx.x; i < C * DIN; i += 4 * NT) {
    const float4 a = *reinterpret_cast<const float4*>(w + i);
    const float x[4] = {a.x, a.y, a.z, a.w};
    wt.put4(i / DIN, i % DIN, x);
  }
}

// phi of the chunk's 16 tokens of this wave: acc[cb][r] = phi(x_t)_c with
// c = 16cb + 4g + r, t = 16w + r16.  nx = |x_t|^2 of that token.
// sc = 1 / sqrt(number of features of the whole map).
template <typename T, int DIN, int C>
__device__ __forceinline__ void rf_tiles(const Planes<FPrec<T>::W, C, DIN>& wt, const Planes<FPrec<T>::X, CH, DIN>& xt,
                                         float nx, int w, int r16, int g, f32x4_t* acc, float sc) {
  using P = FPrec<T>;
  Frag<P::X> xf[DIN / 32];
#pragma unroll
  for (int s = 0; s < DIN / 32; ++s) xf[s] = xt.template frag<P::X>(16 * w + r16, 32 * s, g);
#pragma unroll
  for (int cb = 0; cb < C / 16; ++cb) {
    f32x4_t a = zero4();
#pragma unroll
    for (int s = 0; s < DIN / 32; ++s)
      mmaf<P::W, P::X>(a, wt.template frag<P::W>(16 * cb + r16, 32 * s, g), xf[s]);
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = __builtin_amdgcn_exp2f((a[r] - 0.5f * nx) * 1.4426950408889634f) * sc;
    acc[cb] = a;
  }
}

// Stage a chunk's X rows (already in registers) and return |x_t|^2 for
// token t = 16w + r16.
template <typename T, int DIN>
__device__ __forceinline__ float stage_x(Planes<FPrec<T>::X, CH, DIN>& xt, float* snx, const RowBuf<T, CH, DIN>& bx) {
  bx.stage_values(xt);
  __syncthreads();
  const int t = threadIdx.x >> 2, part = threadIdx.x & 3;  // four threads per token
  if (t < CH) {
    float v[4], acc = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < DIN / 4; c0 += 4) {
      xt.get4(t, part * (DIN / 4) + c0, v);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc += v[q] * v[q];
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if (part == 0) snx[t] = acc;
  }
  __syncthreads();
  return snx[16 * (threadIdx.x >> 6) + (threadIdx.x & 15)];
}

// Walk chunks ch0 .. ch1-1 of head bh: each chunk's X rows are read into
// registers one chunk ahead (two buffers, alternating), then `body(ci, nx)`
// runs with the chunk staged in xt.
template <typename T, int DIN, typename Body>
__device__ __forceinline__ void walk_chunks(Planes<FPrec<T>::X, CH, DIN>& xt, float* snx, const T* Xh, int N,
                                            int ch0, int ch1, Body&& body) {
  RowBuf<T, CH, DIN> b0, b1;
  b0.load(Xh + (size_t)ch0 * CH * DIN, min(CH, N - ch0 * CH));
  auto one = [&](RowBuf<T, CH, DIN>& cur, RowBuf<T, CH, DIN>& nxt, int ci) {
    if (ci + 1 < ch1) nxt.load(Xh + (size_t)(ci + 1) * CH * DIN, min(CH, N - (ci + 1) * CH));
    if (ci > ch0) __syncthreads();  // the previous chunk's reads of xt and snx are done
    body(ci, stage_x<T, DIN>(xt, snx, cur));
  };
  for (int ci = ch0; ci < ch1; ci += 2) {
    one(b0, b1, ci);
    if (ci + 1 < ch1) one(b1, b0, ci + 1);
  }
}

// Random features of `cpw` consecutive 64-token chunks of one head per
// workgroup (W staged once for all of them).  A map of ns > 1 slices of C =
// 64 features (la_wide.h) runs one workgroup per slice: slice s of head bh
// takes rows 64 s .. 64 s + 63 of the head's projection and writes the
// feature-sliced output [bh][s][n][64]; with ns = 1 that is the plain
// [bh][n][C].
template <typename T, int DIN, int C>
__global__ __launch_bounds__(NT) void k_feat_rf(const T* __restrict__ X, const float* __restrict__ W,
                                                 T* __restrict__ Phi, int N, int H, int cpw, int ns, float sc) {
  using P = FPrec<T>;
  __shared__ Planes<P::W, C, DIN> wt;
  __shared__ Planes<P::X, CH, DIN> xt;
  __shared__ alignas(16) float snx[CH];
  const int nch = (N + CH - 1) / CH, ngr = (nch + cpw - 1) / cpw;
  const int bhs = blockIdx.x / ngr, ch0 = (blockIdx.x % ngr) * cpw, ch1 = min(nch, ch0 + cpw);
  const int bh = bhs / ns, sl = bhs % ns;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  stage_w<P::W, C, DIN>(wt, W + ((size_t)(bh % H) * ns + sl) * C * DIN);
  const int t = 16 * w + r16;
  walk_chunks<T, DIN>(xt, snx, X + (size_t)bh * N * DIN, N, ch0, ch1, [&](int ci, float nx) {
    const int c0 = ci * CH;
    f32x4_t acc[C / 16];
    rf_tiles<T, DIN, C>(wt, xt, nx, w, r16, g, acc, sc);
    if (t < N - c0) {
#pragma unroll
      for (int cb = 0; cb < C / 16; ++cb) {
        const float o[4] = {acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]};
        IO<T>::store4(Phi + ((size_t)bhs * N + c0 + t) * C + 16 * cb + 4 * g, o);
      }
    }
  });
}

// dX = W^T (dPhi * phi) - x (dPhi . phi) for `cpw` consecutive 64-token chunks
// of one head per workgroup.
template <typename T, int DIN, int C>
__global__ __launch_bounds__(NT) void k_feat_rf_vjp(const T* __restrict__ X, const float* __restrict__ W,
                                                     const T* __restrict__ dPhi, T* __restrict__ dX, int N, int H,
                                                     int cpw) {
  using P = FPrec<T>;
  __shared__ Planes<P::W, C, DIN> wt;
  __shared__ Planes<P::X, CH, DIN> xt;
  __shared__ alignas(16) float snx[CH];
  const int nch = (N + CH - 1) / CH, ngr = (nch + cpw - 1) / cpw;
  const int bh = blockIdx.x / ngr, ch0 = (blockIdx.x % ngr) * cpw, ch1 = min(nch, ch0 + cpw);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  stage_w<P::W, C, DIN>(wt, W + (size_t)(bh % H) * C * DIN);
  const int t = 16 * w + r16;
  walk_chunks<T, DIN>(xt, snx, X + (size_t)bh * N * DIN, N, ch0, ch1, [&](int ci, float nx) {
    const int c0 = ci * CH;
    const bool ok = t < N - c0;
    // dPhi of the wave's token, four consecutive features per lane, read
    // before the projection so that the loads overlap it
    float d[C / 16][4];
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb) {
      d[cb][0] = d[cb][1] = d[cb][2] = d[cb][3] = 0.f;
      if (ok) {
        if constexpr (sizeof(T) == 4) {
          const float4 a = *reinterpret_cast<const float4*>(dPhi + ((size_t)bh * N + c0 + t) * C + 16 * cb + 4 * g);
          d[cb][0] = a.x; d[cb][1] = a.y; d[cb][2] = a.z; d[cb][3] = a.w;
        } else {
          const uint2 u = *reinterpret_cast<const uint2*>(dPhi + ((size_t)bh * N + c0 + t) * C + 16 * cb + 4 * g);
          d[cb][0] = lo2f(u.x); d[cb][1] = hi2f(u.x); d[cb][2] = lo2f(u.y); d[cb][3] = hi2f(u.y);
        }
      }
    }
    f32x4_t acc[C / 16];
    rf_tiles<T, DIN, C>(wt, xt, nx, w, r16, g, acc, 1.f / sqrtf((float)C));
    // G = dPhi * phi in the same layout, and its sum over the features
    float sg = 0.f;
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[cb][r] *= d[cb][r];
        sg += acc[cb][r];
      }
    }
    sg = sum_over_g(sg);
    Frag<P::G> gf[C / 32];
#pragma unroll
    for (int p = 0; p < C / 32; ++p) gf[p] = acc2frag<P::G>(acc[2 * p], acc[2 * p + 1]);
#pragma unroll
    for (int d0 = 0; d0 < DIN / 16; ++d0) {
      f32x4_t a = zero4();
#pragma unroll
      for (int p = 0; p < C / 32; ++p) mmaf<P::W, P::G>(a, wt.template tfrag_acc<P::W>(32 * p, 16 * d0, g, r16), gf[p]);
      float xv[4];
      xt.get4(t, 16 * d0 + 4 * g, xv);
      if (ok) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = a[r] - xv[r] * sg;
        IO<T>::store4(dX + ((size_t)bh * N + c0 + t) * DIN + 16 * d0 + 4 * g, o);
      }
    }
  });
}

// Degree-2 polynomial features, one thread per token (rows = B H N).
template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (sizeof(T) == 4)
    return *reinterpret_cast<const float*>(p);
  else
    return bf2f(*reinterpret_cast<const bf16_t*>(p));
}
template <typename T>
__device__ __forceinline__ void st1(T* p, float x) {
  if constexpr (sizeof(T) == 4)
    *reinterpret_cast<float*>(p) = x;
  else
    *reinterpret_cast<bf16_t*>(p) = f2bf(x);
}

template <typename T, int C>
__global__ __launch_bounds__(NT) void k_feat_poly2(const T* __restrict__ X, T* __restrict__ Phi, long rows, int din) {
  const long r = (long)blockIdx.x * NT + threadIdx.x;
  if (r >= rows) return;
  float x[8];
  for (int a = 0; a < din; ++a) x[a] = ld1(X + r * din + a);
  float f[C];
#pragma unroll
  for (int c = 0; c < C; ++c) f[c] = 0.f;
  f[0] = 1.f;
  for (int a = 0; a < din; ++a) {
    f[1 + a] = x[a];
    for (int b = 0; b < din; ++b) f[1 + din + a * din + b] = x[a] * x[b];
  }
#pragma unroll
  for (int c = 0; c < C; c += 4) IO<T>::store4(Phi + r * C + c, &f[c]);
}

template <typename T, int C>
__global__ __launch_bounds__(NT) void k_feat_poly2_vjp(const T* __restrict__ X, const T* __restrict__ dPhi,
                                                        T* __restrict__ dX, long rows, int din) {
  const long r = (long)blockIdx.x * NT + threadIdx.x;
  if (r >= rows) return;
  float x[8], g[C];
  for (int a = 0; a < din; ++a) x[a] = ld1(X + r * din + a);
#pragma unroll
  for (int c = 0; c < C; ++c) g[c] = ld1(dPhi + r * C + c);
  for (int a = 0; a < din; ++a) {
    float acc = g[1 + a];
    for (int b = 0; b < din; ++b) acc += (g[1 + din + a * din + b] + g[1 + din + b * din + a]) * x[b];
    st1(dX + r * din + a, acc);
  }
}

}  // namespace la
