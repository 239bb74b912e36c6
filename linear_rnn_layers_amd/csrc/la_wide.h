// la_wide.h -- wide feature maps: attention on feature vectors of C = 64 ns
// features (ns > 1), e.g. the degree-2 polynomial map of a 32-wide head (C =
// 1 + 32 + 32^2 rounded up to 1088) or a few hundred positive random features
// ("Linear Attention/zh", feature maps; "Transformers are RNNs -- part 2/3",
// section 3.2.1: the polynomial kernel costs O(N D^2 M) and pays off once N
// exceeds D^2).
//
// Layout.  Wide feature vectors are stored feature-sliced: [B, H, ns, N, 64],
// slice s holding features 64 s .. 64 s + 63 of every token.  Each slice is
// then an ordinary 64-feature head of the chunked kernels (la_kernels.h,
// la_bwd2.h), and the B H ns slice heads run side by side, slice head bh
// reading the values of head bh / ns.  The state S [B, H, C, M] is the same
// memory as [B H ns, 64, M] (slice s owns rows 64 s .. 64 s + 63), so states,
// checkpoints and their gradients need no conversion.  A single decode token
// [B, H, C] is its own sliced layout.
//
// Everything that sums over features is split by slices and summed here in a
// fixed order (s = 0 .. ns - 1, so results are reproducible run to run):
//   forward:  num_i = sum_s num_i^(s), den_i = sum_s den_i^(s), O_i = num_i /
//             den_i (eq. 9-12 with phi(q_i) . S_i split over the features);
//   backward: dV_j = sum_s (R^(s)_j)^T phi^(s)(K_j) + ... (eq. 15);
// while dphi(Q) and dphi(K) (eq. 13-14) are slice-local once the pair
// (1/den_i, O_i . dO_i) of the whole head is known.  That pair is formed as
// the 64-feature heads form it, from the backward's own states: a first query
// pass writes every slice's shares phi(Q_i)^T S_i dO_i and phi(Q_i) . Z_i
// (la_bwd2.h, kBqShares), and their sums give den_i and O_i . dO_i = (sum of
// the first) / den_i, consistent with the S_i dO_i and Z_i that the
// quotient rule then cancels against each other (taking O_i . dO_i from the
// forward's O instead would leave the two sides of that cancellation with
// independent rounding).
#pragma once

#include "la_feature.h"

namespace la {

// --------------------------------------------------------------- combine
// O_i = sum_s pnum[bh ns + s][i] / sum_s pden[bh ns + s][i] for the B H N
// tokens; M / 4 threads per token, four values each.  den is optional.
template <typename T, int M>
__global__ __launch_bounds__(NT) void k_wide_combine(const float* __restrict__ pnum, const float* __restrict__ pden,
                                                      T* __restrict__ O, float* __restrict__ den, long rows, int N,
                                                      int ns) {
  constexpr int QPT = M / 4;
  const long id = (long)blockIdx.x * NT + threadIdx.x;
  const long tok = id / QPT;
  if (tok >= rows) return;
  const int m0 = 4 * (int)(id % QPT);
  const long bh = tok / N, n = tok % N;
  const size_t stride = (size_t)N * M;  // between slices of one head
  const float* pn = pnum + ((size_t)bh * ns * N + n) * M + m0;
  const float* pd = pden + (size_t)bh * ns * N + n;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float d = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(pn + s * stride);
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
    d += pd[(size_t)s * N];
  }
  const float inv = 1.f / d;
  float o[4] = {a.x * inv, a.y * inv, a.z * inv, a.w * inv};
  IO<T>::store4(O + (size_t)tok * M + m0, o);
  if (den && m0 == 0) den[tok] = d;
}

// gc[i] = (1 / den_i, O_i . dO_i) from the slices' shares sh[bh ns + s][i] =
// (phi^(s)(Q_i)^T S_i^(s) dO_i, phi^(s)(Q_i) . Z_i^(s)), summed in slice order;
// one thread per token.
__global__ __launch_bounds__(NT) void k_wide_pairs(const float2* __restrict__ sh, float2* __restrict__ gc, long rows,
                                                    int N, int ns) {
  const long tok = (long)blockIdx.x * NT + threadIdx.x;
  if (tok >= rows) return;
  const long bh = tok / N, n = tok % N;
  const float2* p = sh + (size_t)bh * ns * N + n;
  float u = 0.f, z = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float2 x = p[(size_t)s * N];
    u += x.x;
    z += x.y;
  }
  const float inv = 1.f / z;
  gc[tok] = make_float2(inv, u * inv);
}

// dV_j = sum_s pdv[bh ns + s][j] into the storage type.
template <typename T, int M>
__global__ __launch_bounds__(NT) void k_wide_sum(const float* __restrict__ pdv, T* __restrict__ dV, long rows, int N,
                                                  int ns) {
  constexpr int QPT = M / 4;
  const long id = (long)blockIdx.x * NT + threadIdx.x;
  const long tok = id / QPT;
  if (tok >= rows) return;
  const int m0 = 4 * (int)(id % QPT);
  const long bh = tok / N, n = tok % N;
  const size_t stride = (size_t)N * M;
  const float* p = pdv + ((size_t)bh * ns * N + n) * M + m0;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < ns; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(p + s * stride);
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
  }
  float o[4] = {a.x, a.y, a.z, a.w};
  IO<T>::store4(dV + (size_t)tok * M + m0, o);
}

// ---------------------------------------------------------------- decode
// One decode step of a head with a wide state (eq. 16-20): one workgroup per
// head streams the C x M float32 state in coalesced float4 rows (M / 4 lanes
// per state row, 1 KiB per instruction across a wavefront), updates it in
// place and reduces phi(q)^T S over its rows, then over the four wavefronts.
constexpr int kWideMax = 4096;  // widest feature vector (64 slices)

template <typename T, int M>
__global__ __launch_bounds__(NT) void k_decode_wide(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, float* __restrict__ S,
                                                     float* __restrict__ Z, T* __restrict__ y, int C, int fm) {
  constexpr int CPL = M / 4;        // lanes per state row
  constexpr int RPP = NT / CPL;     // state rows per pass of the workgroup
  __shared__ float sq[kWideMax], sk[kWideMax], sv[M];
  __shared__ float red[4][M + 1];
  const int head = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const T* qh = q + (size_t)head * C;
  const T* kh = k + (size_t)head * C;
  float* Zh = Z + (size_t)head * C;
  float dn = 0.f;
  for (int c = tid; c < C; c += NT) {
    const float pq = feat(ld1(qh + c), fm), pk = feat(ld1(kh + c), fm);
    sq[c] = pq;
    sk[c] = pk;
    const float z = Zh[c] + pk;
    Zh[c] = z;
    dn += pq * z;
  }
  if (tid < M) sv[tid] = ld1(v + (size_t)head * M + tid);
  __syncthreads();

  const int m0 = 4 * (tid % CPL), r0 = tid / CPL;
  const float v0 = sv[m0], v1 = sv[m0 + 1], v2 = sv[m0 + 2], v3 = sv[m0 + 3];
  float4* S4 = reinterpret_cast<float4*>(S + (size_t)head * C * M);
  float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
  constexpr int U = 4;  // passes in flight
  for (int d0 = r0; d0 < C; d0 += U * RPP) {
    float4 st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * RPP;
      if (d < C) st[u] = S4[(size_t)d * CPL + tid % CPL];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * RPP;
      if (d < C) {
        const float pk = sk[d], pq = sq[d];
        float4 s = st[u];
        s.x += pk * v0;
        s.y += pk * v1;
        s.z += pk * v2;
        s.w += pk * v3;
        S4[(size_t)d * CPL + tid % CPL] = s;
        y0 += pq * s.x;
        y1 += pq * s.y;
        y2 += pq * s.z;
        y3 += pq * s.w;
      }
    }
  }
  // over the rows of the wavefront (lanes with the same column group), then over the wavefronts
#pragma unroll
  for (int off = CPL; off < 64; off <<= 1) {
    y0 += __shfl_xor(y0, off, 64);
    y1 += __shfl_xor(y1, off, 64);
    y2 += __shfl_xor(y2, off, 64);
    y3 += __shfl_xor(y3, off, 64);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dn += __shfl_xor(dn, off, 64);
  if (l < CPL) {
    red[w][4 * l] = y0;
    red[w][4 * l + 1] = y1;
    red[w][4 * l + 2] = y2;
    red[w][4 * l + 3] = y3;
  }
  if (l == 0) red[w][M] = dn;
  __syncthreads();
  if (tid < CPL) {
    const float den = red[0][M] + red[1][M] + red[2][M] + red[3][M];
    const float inv = 1.f / den;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (red[0][4 * tid + e] + red[1][4 * tid + e] + red[2][4 * tid + e] +
                                        red[3][4 * tid + e]) * inv;
    IO<T>::store4(y + (size_t)head * M + 4 * tid, o);
  }
}

// ------------------------------------------------------ random features
// Vector-Jacobian product of wide random features (C = 64 ns): dX = sum_c
// dPhi_c phi_c (w_c - x) sums over every slice.  A workgroup owns CPW
// consecutive chunks of one head with their X staged once; it walks the
// slices, staging W's 64 rows of each, recomputes the slice's phi (float32),
// forms G = dPhi * phi and accumulates W_s^T G and sum_c G_c in registers;
// dX = W^T G - x sum_c G_c at the end.
template <typename T, int DIN, int CPW>
__global__ __launch_bounds__(NT) void k_feat_rf_vjp_wide(const T* __restrict__ X, const float* __restrict__ W,
                                                          const T* __restrict__ dPhi, T* __restrict__ dX, int N,
                                                          int H, int ns, float sc) {
  using P = FPrec<T>;
  constexpr int C = 64;  // features per slice
  __shared__ Planes<P::W, C, DIN> wt;
  __shared__ Planes<P::X, CH * CPW, DIN> xt;
  __shared__ alignas(16) float snx[CH * CPW];
  const int nch = (N + CH - 1) / CH, ngr = (nch + CPW - 1) / CPW;
  const int bh = blockIdx.x / ngr, ch0 = (blockIdx.x % ngr) * CPW;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int n0 = ch0 * CH, nrows = min(CH * CPW, N - n0);
  const T* Xh = X + ((size_t)bh * N + n0) * DIN;
  // X of the workgroup's tokens (zero past the end) and |x|^2 per token
  for (int e = tid; e < CH * CPW * DIN / 4; e += NT) {
    const int row = e / (DIN / 4), col = 4 * (e % (DIN / 4));
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (row < nrows) IO<T>::load4(Xh + (size_t)row * DIN + col, x);
    xt.put4(row, col, x);
  }
  __syncthreads();
  for (int row = tid; row < CH * CPW; row += NT) {
    float acc = 0.f, x[4];
    for (int c0 = 0; c0 < DIN; c0 += 4) {
      xt.get4(row, c0, x);
      acc += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
    snx[row] = acc;
  }
  f32x4_t dx[CPW][DIN / 16];
  float sg[CPW];
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    sg[ci] = 0.f;
#pragma unroll
    for (int d0 = 0; d0 < DIN / 16; ++d0) dx[ci][d0] = zero4();
  }
  for (int s = 0; s < ns; ++s) {
    __syncthreads();  // the previous slice's reads of wt are done (and, at s = 0, X is staged)
    stage_w<P::W, C, DIN>(wt, W + ((size_t)(bh % H) * ns + s) * C * DIN);
    __syncthreads();
    const T* dPs = dPhi + ((size_t)bh * ns + s) * N * C;
#pragma unroll
    for (int ci = 0; ci < CPW; ++ci) {
      const int row = CH * ci + 16 * w + r16;  // this lane's token within the workgroup
      const bool ok = row < nrows;
      float d[C / 16][4];
#pragma unroll
      for (int cb = 0; cb < C / 16; ++cb) {
        d[cb][0] = d[cb][1] = d[cb][2] = d[cb][3] = 0.f;
        if (ok) IO<T>::load4(dPs + (size_t)(n0 + row) * C + 16 * cb + 4 * g, d[cb]);
      }
      Frag<P::X> xf[DIN / 32];
#pragma unroll
      for (int t = 0; t < DIN / 32; ++t) xf[t] = xt.template frag<P::X>(row, 32 * t, g);
      const float nx = snx[row];
      f32x4_t acc[C / 16];
      float gs = 0.f;
#pragma unroll
      for (int cb = 0; cb < C / 16; ++cb) {
        f32x4_t a = zero4();
#pragma unroll
        for (int t = 0; t < DIN / 32; ++t) mmaf<P::W, P::X>(a, wt.template frag<P::W>(16 * cb + r16, 32 * t, g), xf[t]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = __builtin_amdgcn_exp2f((a[r] - 0.5f * nx) * 1.4426950408889634f) * sc * d[cb][r];
          gs += a[r];
        }
        acc[cb] = a;
      }
      sg[ci] += sum_over_g(gs);
      Frag<P::G> gf[C / 32];
#pragma unroll
      for (int p = 0; p < C / 32; ++p) gf[p] = acc2frag<P::G>(acc[2 * p], acc[2 * p + 1]);
#pragma unroll
      for (int d0 = 0; d0 < DIN / 16; ++d0) {
#pragma unroll
        for (int p = 0; p < C / 32; ++p)
          mmaf<P::W, P::G>(dx[ci][d0], wt.template tfrag_acc<P::W>(32 * p, 16 * d0, g, r16), gf[p]);
      }
    }
  }
#pragma unroll
  for (int ci = 0; ci < CPW; ++ci) {
    const int row = CH * ci + 16 * w + r16;
    if (row >= nrows) continue;
#pragma unroll
    for (int d0 = 0; d0 < DIN / 16; ++d0) {
      float xv[4], o[4];
      xt.get4(row, 16 * d0 + 4 * g, xv);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = dx[ci][d0][r] - xv[r] * sg[ci];
      IO<T>::store4(dX + ((size_t)bh * N + n0 + row) * DIN + 16 * d0 + 4 * g, o);
    }
  }
}

// ------------------------------------------------- polynomial features
// Feature c of the degree-2 map of x (Din values): 1, then x_1 .. x_Din, then
// x_a x_b (a-major), then zeros.  (a, b) of a quadratic feature i = c - 1 -
// Din comes from a float reciprocal: (i + 1/2) / Din lies at least 1 / (2 Din)
// from an integer, far beyond the rounding of (i + 1/2) * (1/Din) for i <
// 4096, so the truncation is the exact quotient.
struct Poly2Index {
  int din;
  float rdin;
  __device__ explicit Poly2Index(int d) : din(d), rdin(1.f / (float)d) {}
  // kind: 0 the constant, 1 linear (a), 2 quadratic (a, b), 3 padding
  __device__ __forceinline__ int at(int c, int& a, int& b) const {
    if (c == 0) return 0;
    if (c <= din) {
      a = c - 1;
      return 1;
    }
    const int i = c - 1 - din;
    if (i >= din * din) return 3;
    a = (int)(((float)i + 0.5f) * rdin);
    b = i - a * din;
    return 2;
  }
};

// 64 tokens of one head per workgroup, every slice: X staged once, each
// 16-byte vector of the feature-sliced output (8 bf16 or 4 float32 features
// of one token) formed in registers and written whole.
template <typename T>
__global__ __launch_bounds__(NT) void k_feat_poly2_wide(const T* __restrict__ X, T* __restrict__ Phi, int N, int din,
                                                         int ns) {
  constexpr int E = IO<T>::E;  // features per 16-byte vector
  constexpr int PR = 64 / E;   // vectors per token row of a slice
  __shared__ float xs[CH][64 + 1];
  const int ntb = (N + CH - 1) / CH;
  const int bh = blockIdx.x / ntb, n0 = (blockIdx.x % ntb) * CH;
  const int tid = threadIdx.x, nrows = min(CH, N - n0);
  const Poly2Index ix(din);
  for (int e = tid; e < CH * din; e += NT) {
    const int row = e / din, a = e % din;
    xs[row][a] = row < nrows ? ld1(X + ((size_t)bh * N + n0 + row) * din + a) : 0.f;
  }
  __syncthreads();
  for (int p = tid; p < ns * CH * PR; p += NT) {
    const int s = p / (CH * PR), r = p % (CH * PR), tt = r / PR, c0 = 64 * s + (r % PR) * E;
    if (tt >= nrows) continue;
    float f[E];
    // (a, b) of the vector's first quadratic feature from the reciprocal, then stepped along the row
    const int q0 = c0 - 1 - din;  // index among the quadratic features (negative: the head of the map)
    int a = 0, b = 0;
    if (q0 > 0) ix.at(c0, a, b);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = c0 + e, q = q0 + e;
      if (q < 0) {
        f[e] = c == 0 ? 1.f : xs[tt][c - 1];
      } else {
        if (q == 0) a = b = 0;
        f[e] = q < din * din ? xs[tt][a] * xs[tt][b] : 0.f;
        if (++b == din) {
          b = 0;
          ++a;
        }
      }
    }
    T* out = Phi + (((size_t)bh * ns + s) * N + n0 + tt) * 64 + (r % PR) * E;
#pragma unroll
    for (int q = 0; q < E; q += 4) IO<T>::store4(out + q, f + q);
  }
}

// dX_a = dPhi_(1 + a) + sum_b (G_ab + G_ba) x_b with G_ab = dPhi_(1 + din + a
// din + b): tpw tokens per workgroup (as many as fit a 64 KiB LDS buffer, at
// most 32).  Each token's feature gradient is copied into LDS as one flat row
// of C values in 16-byte vectors (slice by slice; each slice's rows of
// consecutive tokens are contiguous in memory); then DMAX threads per token,
// one per a, read G's row a (rotated by a, so that the lanes of a wavefront
// fall in different banks) and column a.
constexpr int kPolyVjpLds = 64 << 10;

template <typename T, int DMAX>
__global__ __launch_bounds__(NT) void k_feat_poly2_vjp_wide(const T* __restrict__ X, const T* __restrict__ dPhi,
                                                             T* __restrict__ dX, long rows, int N, int din, int ns,
                                                             int tpw) {
  constexpr int E = IO<T>::E, PR = 64 / E, BATCH = 8, TMAX = 32;
  __shared__ alignas(16) T flat[kPolyVjpLds / sizeof(T)];
  __shared__ float xs[TMAX][DMAX];
  __shared__ long tbase[TMAX];  // element offset of the token's row in slice 0
  const int tid = threadIdx.x, C = 64 * ns;
  const long tok0 = (long)blockIdx.x * tpw;
  const int ntok = (int)min((long)tpw, rows - tok0);
  if (tid < ntok) {
    const long tok = tok0 + tid, bh = tok / N, n = tok % N;
    tbase[tid] = ((long)bh * ns * N + n) * 64;
  }
  for (int e = tid; e < ntok * din; e += NT) {
    const int tt = e / din, a = e % din;
    xs[tt][a] = ld1(X + (size_t)(tok0 + tt) * din + a);
  }
  __syncthreads();
  const int total = ns * ntok * PR;  // 16-byte vectors: (slice, token, vector of the slice row)
  for (int p0 = tid; p0 < total; p0 += NT * BATCH) {
    typename IO<T>::raw v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + u * NT;
      if (p < total) {
        const int s = p / (ntok * PR), r = p % (ntok * PR), tt = r / PR;
        v[u] = IO<T>::load_raw(dPhi + tbase[tt] + (size_t)s * N * 64 + (r % PR) * E);
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + u * NT;
      if (p < total) {
        const int s = p / (ntok * PR), r = p % (ntok * PR), tt = r / PR;
        *reinterpret_cast<typename IO<T>::raw*>(&flat[tt * C + 64 * s + (r % PR) * E]) = v[u];
      }
    }
  }
  __syncthreads();
  for (int q = tid; q < ntok * DMAX; q += NT) {
    const int tt = q / DMAX, a = q % DMAX;
    if (a >= din) continue;
    const T* f = flat + tt * C;
    const T* g = f + 1 + din;  // G, row-major din x din
    float acc = ld1(f + 1 + a);
    int b = a;  // row a visited from b = a on
    for (int k = 0; k < din; ++k) {
      acc += ld1(g + a * din + b) * xs[tt][b] + ld1(g + k * din + a) * xs[tt][k];
      b = b + 1 == din ? 0 : b + 1;
    }
    st1(dX + (size_t)(tok0 + tt) * din + a, acc);
  }
}

}  // namespace la
