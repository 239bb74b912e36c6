// la_kernels.h -- gfx950 kernels for causal linear attention, phi = elu + 1.
//
// Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
// Attention -- part 2/3", eq. 7-20; non-causal form: reading notes on the same
// paper, section 3.2 eq. 5-6; chunked evaluation of the causal sums:
// "Linear Attention/zh", training / parallel form (cut the sequence into
// blocks, quadratic masked attention inside a block, linear state updates
// between blocks).
//
// Work decomposition.  Each (batch*head) sequence is cut into segments of L
// tokens (a multiple of 64); one workgroup of four wavefronts owns one (head,
// segment) and walks its chunks in order, carrying the state (S, Z) -- in the
// backward also the reverse state (R, r) -- in registers, with the chunk's
// operands staged once per chunk in LDS as bf16 planes (la_device.h) while
// the next chunk's global reads are in flight.  A segment's start state is the
// sum, in a fixed order, of the aggregates of the segments before it (after
// it, for the reverse state), written by a separate aggregate pass: results
// are bitwise reproducible and no workgroup waits for another.
//
// Inside a chunk every contraction is a 16x16 MFMA tile product; wave w owns
// the 16 tokens 16w..16w+15 of a 64-token chunk.
#include "la_device.h"

namespace la {

constexpr int CH = 64;  // forward chunk

// Planes per staged operand and per product for each storage type.
// bf16 I/O: inputs V, dO are exact in one plane; computed operands use one
// plane where the result only needs bf16 accuracy and two where a state
// accumulates or a later subtraction cancels.  float32 I/O: two planes where
// about 2^-16 suffices, three (float32 level) for the query-gradient path and
// the carried state, whose errors the cancellation in dQ would amplify.
template <typename T>
struct Prec;
template <>
struct Prec<bf16_t> {
  // forward: phi(Q) tok, phi(K) tok, phi(K) feat, V feat, S^T, A (accumulators)
  static constexpr int FQ = 1, FK = 1, FKF = 2, FV = 1, FS = 1, FA = 1;
  // backward staging
  static constexpr int BQT = 2, BQF = 2, BKT = 2, BKF = 2, BVT = 1, BDO = 1, BG = 2, BS = 2, BR = 2;
  // backward products
  static constexpr int dS_a = 1, dS_b = 2, Bt = 1, U1_a = 2, U1_b = 1, U2 = 2, Zc = 2, dR = 2, At = 2, Wt = 1,
                       dK = 2, KR_a = 2, KR_b = 1, dV = 2, VR = 2;
};
template <>
struct Prec<float> {
  static constexpr int FQ = 2, FK = 2, FKF = 3, FV = 3, FS = 2, FA = 2;
  static constexpr int BQT = 3, BQF = 3, BKT = 2, BKF = 3, BVT = 3, BDO = 3, BG = 2, BS = 3, BR = 2;
  // g_i.V_j + c_i cancels where V_j = O_i, so dO.V and its product with
  // phi(Q) are taken at float32 level too (bf16 inputs make dO.V exact).
  static constexpr int dS_a = 3, dS_b = 3, Bt = 3, U1_a = 3, U1_b = 3, U2 = 3, Zc = 3, dR = 2, At = 2, Wt = 3,
                       dK = 3, KR_a = 2, KR_b = 2, dV = 2, VR = 2;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Backward chunk: 64 tokens, or 32 when float32 I/O with a 64-wide dimension
// would not fit the planes in LDS.
template <typename T, int D, int M>
struct BwdChunk {
  static constexpr int value = (sizeof(T) == 4 && (D == 64 || M == 64)) ? 32 : 64;
};

// Sum of state vectors in tile layout: lane holds S^T[16mb + 4g + r][16db + r16]
// of tile t = w + 4k; reads S[d][m] row-major states base + p * stride, p in [p0, p1).
template <int D, int M, int NTW>
__device__ __forceinline__ void sum_states_tiles(f32x4_t* acc, const float* base, long stride, int p0, int p1,
                                                 int w, int r16, int g) {
  constexpr int DB = D / 16;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    const float* e = base + (16 * db + r16) * M + 16 * mb + 4 * g;
    for (int p = p0; p < p1; ++p) {
      const float4 a = *reinterpret_cast<const float4*>(e + (long)p * stride);
      acc[k] += f32x4_t{a.x, a.y, a.z, a.w};
    }
  }
}

// ===================================================================== F1
// Segment aggregates: agg[bh][seg] = ( sum_j phi(K_j) V_j^T  [D][M],
//                                      sum_j phi(K_j)        [D] )
// over the segment's tokens (eq. 10-11 restricted to one segment).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_seg_state(const T* __restrict__ K, const T* __restrict__ V,
                                                   float* __restrict__ agg, int N, int L, int nseg) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  constexpr int NKF = P::FKF, NVF = cmax(P::FV, 1);
  __shared__ Planes<NKF, D, CH> kf;
  __shared__ Planes<NVF, M, CH> vf;
  __shared__ float zpart[4][D];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;

  f32x4_t acc[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();
  float z = 0.f;

  RowBuf<T, CH, D> bk;
  RowBuf<T, CH, M> bv;
  bk.load(Kh + (size_t)t0 * D, min(CH, t1 - t0));
  bv.load(Vh + (size_t)t0 * M, min(CH, t1 - t0));
  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    __syncthreads();
    bk.for_each(nv, [&](int r, int c, const float* x, bool ok) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) kf.put(c + e, r, ok ? phi(x[e]) : 0.f);
    });
    bv.for_each(nv, [&](int r, int c, const float* x, bool) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) vf.put(c + e, r, x[e]);
    });
    if (c0 + CH < t1) {
      bk.load(Kh + (size_t)(c0 + CH) * D, min(CH, t1 - c0 - CH));
      bv.load(Vh + (size_t)(c0 + CH) * M, min(CH, t1 - c0 - CH));
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s)
        mmaf<P::FV, P::FKF>(acc[k], vf.template frag<P::FV>(16 * mb + r16, 32 * s, g),
                            kf.template frag<P::FKF>(16 * db + r16, 32 * s, g));
    }
    {  // Z: each wave sums 16 of the chunk's tokens for every feature
      for (int d = l; d < D; d += 64) {
        float zs = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) zs += kf.get(d, 16 * w + j);
        z += zs;
      }
    }
  }
  if (l < D) zpart[w][l] = z;
  __syncthreads();
  float* out = agg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
        make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
  if (tid < D) out[D * M + tid] = zpart[0][tid] + zpart[1][tid] + zpart[2][tid] + zpart[3][tid];
}

// ===================================================================== F3
// Chunked forward over one segment.
//   causal: for each chunk, A^T = phi(K) phi(Q)^T masked to j <= i (eq. 8),
//     num^T = V^T A^T + S^T phi(Q)^T, den = rowsum(A) + phi(Q).Z, O = num/den
//     (eq. 9-12), then S += phi(K)^T V, Z += colsum phi(K) (eq. 10-11).
//     The start state is (S0, Z0) plus the aggregates of the earlier
//     segments; it is written to the checkpoint, and the last segment writes
//     the final state (checkpoint entry nseg, S_out/Z_out).
//   non-causal: num^T = S^T phi(Q)^T with S, Z the sum of all segment
//     aggregates (eq. 5-6).
template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_fwd(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, T* __restrict__ O, float* __restrict__ den_out,
                                             const float* __restrict__ agg, const float* __restrict__ S0,
                                             const float* __restrict__ Z0, float* __restrict__ ckpt,
                                             float* __restrict__ S_out, float* __restrict__ Z_out, int N, int L,
                                             int nseg) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  constexpr int KR = CAUSAL ? CH : 1, KD = CAUSAL ? D : 1, KM = CAUSAL ? M : 1;
  __shared__ Planes<P::FQ, CH, D> qt;
  __shared__ Planes<P::FK, KR, KD> kt;
  __shared__ Planes<P::FKF, KD, KR> kf;
  __shared__ Planes<P::FV, KM, KR> vf;
  __shared__ Planes<P::FS, M, D> st;  // S^T
  __shared__ float sZ[D];
  __shared__ float zpart[4][D];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;
  T* Oh = O + (size_t)bh * N * M;

  RowBuf<T, CH, D> bq, bk;
  RowBuf<T, CH, M> bv;
  bq.load(Qh + (size_t)t0 * D, min(CH, t1 - t0));
  if constexpr (CAUSAL) {
    bk.load(Kh + (size_t)t0 * D, min(CH, t1 - t0));
    bv.load(Vh + (size_t)t0 * M, min(CH, t1 - t0));
  }

  // ---- start state
  f32x4_t accS[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) accS[k] = zero4();
  const float* aggh = agg ? agg + (size_t)bh * nseg * SV : nullptr;
  const int pend = CAUSAL ? seg : nseg;
  if (S0) sum_states_tiles<D, M, NTW>(accS, S0 + (size_t)bh * D * M, 0, 0, 1, w, r16, g);
  if (aggh) sum_states_tiles<D, M, NTW>(accS, aggh, SV, 0, pend, w, r16, g);
  if (tid < D) {
    float z = Z0 ? Z0[(size_t)bh * D + tid] : 0.f;
    if (aggh)
      for (int p = 0; p < pend; ++p) z += aggh[(size_t)p * SV + D * M + tid];
    sZ[tid] = z;
  }
  if (CAUSAL && ckpt) {
    float* ck = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
      *reinterpret_cast<float4*>(ck + (16 * db + r16) * M + 16 * mb + 4 * g) =
          make_float4(accS[k][0], accS[k][1], accS[k][2], accS[k][3]);
    }
    if (tid < D) ck[D * M + tid] = sZ[tid];
  }
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
    for (int r = 0; r < 4; ++r) st.put(16 * mb + 4 * g + r, 16 * db + r16, accS[k][r]);
  }

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    const int nn = min(CH, t1 - c0 - CH);  // rows of the next chunk (<= 0: none)
    __syncthreads();
    bq.for_each(nv, [&](int r, int c, const float* x, bool ok) {
      float p[IO<T>::E];
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) p[e] = ok ? phi(x[e]) : 0.f;
      qt.template putrow<IO<T>::E>(r, c, p);
    });
    if (nn > 0) bq.load(Qh + (size_t)(c0 + CH) * D, nn);
    if constexpr (CAUSAL) {
      bk.for_each(nv, [&](int r, int c, const float* x, bool ok) {
        float p[IO<T>::E];
#pragma unroll
        for (int e = 0; e < IO<T>::E; ++e) {
          p[e] = ok ? phi(x[e]) : 0.f;
          kf.put(c + e, r, p[e]);
        }
        kt.template putrow<IO<T>::E>(r, c, p);
      });
      bv.for_each(nv, [&](int r, int c, const float* x, bool) {
#pragma unroll
        for (int e = 0; e < IO<T>::E; ++e) vf.put(c + e, r, x[e]);
      });
      if (nn > 0) {
        bk.load(Kh + (size_t)(c0 + CH) * D, nn);
        bv.load(Vh + (size_t)(c0 + CH) * M, nn);
      }
    }
    __syncthreads();

    const int il = 16 * w + r16;
    Frag<P::FQ> qf[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = qt.template frag<P::FQ>(il, 32 * s, g);

    float dp = 0.f;
    Frag<P::FA> af[2];
    if constexpr (CAUSAL) {
      f32x4_t accA[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) mmaf<P::FK, P::FQ>(a, kt.template frag<P::FK>(16 * jb + r16, 32 * s, g), qf[s]);
          if (jb == w) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * g + r > r16) a[r] = 0.f;  // A^T[j][i] with j > i is masked (eq. 8)
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) dp += a[r];
        }
        accA[jb] = a;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) af[p] = acc2frag<P::FA>(accA[2 * p], accA[2 * p + 1]);
    }
#pragma unroll
    for (int dd = 0; dd < D / 4; dd += 4) {
      float qv[4];
      qt.get4(il, g * (D / 4) + dd, qv);
#pragma unroll
      for (int q = 0; q < 4; ++q) dp += qv[q] * sZ[g * (D / 4) + dd + q];
    }
    dp = sum_over_g(dp);
    const float inv = 1.f / dp;
    const bool row_ok = il < nv;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t acc = zero4();
      if constexpr (CAUSAL) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p <= w) mmaf<P::FV, P::FA>(acc, vf.template frag_acc<P::FV>(16 * mb + r16, 32 * p, g), af[p]);
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mmaf<P::FS, P::FQ>(acc, st.template frag<P::FS>(16 * mb + r16, 32 * s, g), qf[s]);
      if (row_ok) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[r] * inv;
        IO<T>::store4(Oh + (size_t)(c0 + il) * M + 16 * mb + 4 * g, o);
      }
    }
    if (den_out && g == 0 && row_ok) den_out[(size_t)bh * N + c0 + il] = dp;

    if constexpr (CAUSAL) {
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
        for (int s = 0; s < CH / 32; ++s)
          mmaf<P::FV, P::FKF>(accS[k], vf.template frag<P::FV>(16 * mb + r16, 32 * s, g),
                              kf.template frag<P::FKF>(16 * db + r16, 32 * s, g));
      }
      for (int d = l; d < D; d += 64) {
        float zs = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) zs += kf.get(d, 16 * w + j);
        zpart[w][d] = zs;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
        for (int r = 0; r < 4; ++r) st.put(16 * mb + 4 * g + r, 16 * db + r16, accS[k][r]);
      }
      if (tid < D) sZ[tid] += zpart[0][tid] + zpart[1][tid] + zpart[2][tid] + zpart[3][tid];
    }
  }
  if constexpr (CAUSAL) {
    if (seg == nseg - 1 && (S_out || ckpt)) {
      __syncthreads();
      float* ck = ckpt ? ckpt + ((size_t)bh * (nseg + 1) + nseg) * SV : nullptr;
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
        const float4 v4 = make_float4(accS[k][0], accS[k][1], accS[k][2], accS[k][3]);
        const int off = (16 * db + r16) * M + 16 * mb + 4 * g;
        if (S_out) *reinterpret_cast<float4*>(S_out + (size_t)bh * D * M + off) = v4;
        if (ck) *reinterpret_cast<float4*>(ck + off) = v4;
      }
      if (tid < D) {
        if (Z_out) Z_out[(size_t)bh * D + tid] = sZ[tid];
        if (ck) ck[D * M + tid] = sZ[tid];
      }
    }
  }
}

// Checkpoint from segment aggregates (used when the backward is called without
// the forward's checkpoint): ckpt[bh][s] = init + sum_{t<s} agg[bh][t], s = 0..nseg.
template <int D, int M>
__global__ __launch_bounds__(NT) void k_scan_states(const float* __restrict__ agg, const float* __restrict__ S0,
                                                     const float* __restrict__ Z0, float* __restrict__ ckpt, int nseg) {
  constexpr int SV = D * M + D;
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NT + threadIdx.x;
  if (e >= SV) return;
  float run = 0.f;
  if (e < D * M) {
    if (S0) run = S0[(size_t)bh * D * M + e];
  } else {
    if (Z0) run = Z0[(size_t)bh * D + (e - D * M)];
  }
  for (int s = 0; s < nseg; ++s) {
    ckpt[((size_t)bh * (nseg + 1) + s) * SV + e] = run;
    run += agg[((size_t)bh * nseg + s) * SV + e];
  }
  ckpt[((size_t)bh * (nseg + 1) + nseg) * SV + e] = run;
}

// Final state for an empty sequence (N = 0): S_out = S0, checkpoint = [S0].
template <int D, int M>
__global__ __launch_bounds__(NT) void k_state_copy(const float* __restrict__ S0, const float* __restrict__ Z0,
                                                    float* __restrict__ ckpt, float* __restrict__ S_out,
                                                    float* __restrict__ Z_out) {
  constexpr int SV = D * M + D;
  const int bh = blockIdx.x;
  for (int e = threadIdx.x; e < SV; e += NT) {
    const float v = e < D * M ? (S0 ? S0[(size_t)bh * D * M + e] : 0.f) : (Z0 ? Z0[(size_t)bh * D + e - D * M] : 0.f);
    if (ckpt) ckpt[(size_t)bh * SV + e] = v;
    if (S_out) {
      if (e < D * M)
        S_out[(size_t)bh * D * M + e] = v;
      else
        Z_out[(size_t)bh * D + e - D * M] = v;
    }
  }
}

// ===================================================================== B1
// Segment aggregates of the reverse state: ragg[bh][seg] =
//   ( R = sum_i phi(Q_i) g_i^T [D][M],  r = sum_i c_i phi(Q_i) [D] )
// i.e. the backward-running sums of eq. 14-15 over one segment, with the
// upstream [g, c] of the numerator and the denominator (g_i = dO_i / den_i,
// c_i = -(dO_i . O_i) / den_i), taken from the forward's O and den.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_seg_rstate(const T* __restrict__ Q, const T* __restrict__ O,
                                                    const float* __restrict__ den, const T* __restrict__ dO,
                                                    float* __restrict__ ragg, int N, int L, int nseg) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  constexpr int E = IO<T>::E, PRM = M / E;
  __shared__ Planes<P::dR, D, CH> qf;  // phi(Q), feature-major
  __shared__ Planes<P::dR, M, CH> gf;  // g, feature-major
  __shared__ float sC[CH];
  __shared__ float rpart[4][D];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Oh = O + (size_t)bh * N * M;
  const T* dOh = dO + (size_t)bh * N * M;
  const float* denh = den + (size_t)bh * N;

  f32x4_t acc[NTW];  // R^T tiles: [16mb + 4g + r][16db + r16]
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();
  float rr = 0.f;

  RowBuf<T, CH, D> bq;
  RowBuf<T, CH, M> bo, bd;
  bq.load(Qh + (size_t)t0 * D, min(CH, t1 - t0));
  bo.load(Oh + (size_t)t0 * M, min(CH, t1 - t0));
  bd.load(dOh + (size_t)t0 * M, min(CH, t1 - t0));
  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    const int nn = min(CH, t1 - c0 - CH);
    __syncthreads();
    bq.for_each(nv, [&](int r, int c, const float* x, bool ok) {
#pragma unroll
      for (int e = 0; e < E; ++e) qf.put(c + e, r, ok ? phi(x[e]) : 0.f);
    });
    // g and c need den (per row) and dO . O (a row reduction over PRM lanes)
#pragma unroll
    for (int i = 0; i < RowBuf<T, CH, M>::CNT; ++i) {
      const int v = tid + i * NT;
      const int r = v / PRM, c = (v % PRM) * E;
      float xo[E], xd[E];
      IO<T>::unpack(bo.r[i], xo);
      IO<T>::unpack(bd.r[i], xd);
      const float dn = r < nv ? denh[c0 + r] : 1.f;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part += xd[e] * xo[e];
#pragma unroll
      for (int off = PRM / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
      const float inv = 1.f / dn;
#pragma unroll
      for (int e = 0; e < E; ++e) gf.put(c + e, r, xd[e] * inv);
      if (c == 0) sC[r] = -part * inv;
    }
    if (nn > 0) {
      bq.load(Qh + (size_t)(c0 + CH) * D, nn);
      bo.load(Oh + (size_t)(c0 + CH) * M, nn);
      bd.load(dOh + (size_t)(c0 + CH) * M, nn);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s)
        mmaf<P::dR, P::dR>(acc[k], gf.template frag<P::dR>(16 * mb + r16, 32 * s, g),
                           qf.template frag<P::dR>(16 * db + r16, 32 * s, g));
    }
    for (int d = l; d < D; d += 64) {
      float s_ = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s_ += sC[16 * w + i] * qf.get(d, 16 * w + i);
      rr += s_;
    }
  }
  if (l < D) rpart[w][l] = rr;
  __syncthreads();
  float* out = ragg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
        make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
  if (tid < D) out[D * M + tid] = rpart[0][tid] + rpart[1][tid] + rpart[2][tid] + rpart[3][tid];
}

// ===================================================================== B3
// Backward over one segment, chunks in reverse order.  Registers carry
//   S (forward sum of phi(K) V^T, eq. 13), walked backwards from the
//     segment's end state by removing each chunk's contribution (the first
//     chunk restarts from the segment's start state), and
//   R (backward sum of phi(Q) g^T, eq. 14-15) from the sum of the later
//     segments' aggregates.
// Per chunk, the waves produce
//   dQ: with u_i = S_i dO_i, Z_i the inclusive normaliser, den_i =
//     phi(Q_i).Z_i and O_i.dO_i = phi(Q_i).u_i / den_i (both recomputed
//     here), dphiQ_i = (u_i - Z_i (O_i.dO_i)) / den_i, which is eq. 13's
//     S_i g_i plus the denominator's share c_i Z_i (g_i = dO_i / den_i,
//     c_i = -(O_i.dO_i) / den_i);
//   dK, dV: dphiK_j = sum_{i>=j} phi(Q_i)(g_i.V_j + c_i) + R V_j + r,
//     dV_j = sum_{i>=j} g_i (phi(Q_i).phi(K_j)) + R^T phi(K_j)
//     (eq. 14-15 on [V, 1] with upstream [g, c]);
// and the chain rule through phi.  The stored O and den are not read: the
// recomputed den_i and O_i.dO_i are exact to float32, so g_i.V_j + c_i
// cancels exactly where V_j = O_i even for bf16 storage.
// With 64-token chunks wave w handles both gradients of tokens 16w..; with
// 32-token chunks waves 0-1 produce dQ and waves 2-3 dK, dV.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_bwd(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, const T* __restrict__ dO,
                                             const float* __restrict__ ckpt, const float* __restrict__ ragg,
                                             T* __restrict__ dQ, T* __restrict__ dK, T* __restrict__ dV, int N, int L,
                                             int nseg) {
  using P = Prec<T>;
  constexpr int CB = BwdChunk<T, D, M>::value;
  constexpr int RB = CB / 16, NPAIR = CB / 32;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  __shared__ Planes<P::BQT, CB, D> qt;  // phi(Q), token-major
  __shared__ Planes<P::BQF, D, CB> qf;  // phi(Q), feature-major
  __shared__ Planes<P::BKT, CB, D> kt;  // phi(K), token-major
  __shared__ Planes<P::BKF, D, CB> kf;  // phi(K), feature-major
  __shared__ Planes<P::BVT, CB, M> vt;  // V, token-major
  __shared__ Planes<P::BDO, CB, M> ot;  // dO, token-major
  __shared__ Planes<P::BG, M, CB> gf;   // g = dO / den, feature-major
  __shared__ Planes<P::BS, D, M> sp;    // S before this chunk, [d][m]
  __shared__ Planes<P::BR, D, M> rp;    // R after this chunk, [d][m]
  __shared__ float sZ[D], sr[D], sDen[CB], sC[CB];
  __shared__ float zpart[4][D];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;
  const bool has_q = RB == 4 || w < 2;
  const bool has_kv = RB == 4 || w >= 2;
  const int qrb = w, kvrb = RB == 4 ? w : w - 2;

  const float* st_start = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
  const float* st_end = st_start + SV;

  const int nchunk = (t1 - t0 + CB - 1) / CB;
  RowBuf<T, CB, D> bq, bk;
  RowBuf<T, CB, M> bv, bd;
  {
    const int c0 = t0 + (nchunk - 1) * CB, nv = min(CB, t1 - c0);
    bq.load(Q + offD + (size_t)c0 * D, nv);
    bk.load(K + offD + (size_t)c0 * D, nv);
    bv.load(V + offM + (size_t)c0 * M, nv);
    bd.load(dO + offM + (size_t)c0 * M, nv);
  }

  f32x4_t accS[NTW], accR[NTW];  // S^T and R^T tiles: [16mb + 4g + r][16db + r16]
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    accS[k] = zero4();
    accR[k] = zero4();
  }
  sum_states_tiles<D, M, NTW>(accS, st_end, 0, 0, 1, w, r16, g);
  const float* raggh = ragg ? ragg + (size_t)bh * nseg * SV : nullptr;
  if (raggh) sum_states_tiles<D, M, NTW>(accR, raggh, SV, seg + 1, nseg, w, r16, g);
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
    for (int r = 0; r < 4; ++r) rp.put(16 * db + r16, 16 * mb + 4 * g + r, accR[k][r]);
  }
  float zcur = 0.f, rcur = 0.f;
  if (tid < D) {
    zcur = st_end[D * M + tid];
    if (raggh)
      for (int p = seg + 1; p < nseg; ++p) rcur += raggh[(size_t)p * SV + D * M + tid];
    sr[tid] = rcur;
  }

  for (int ci = nchunk - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * CB;
    const int nv = min(CB, t1 - c0);
    // ---- stage this chunk from registers, then start reading the previous one
    __syncthreads();
    bq.for_each(nv, [&](int r, int c, const float* x, bool ok) {
      float p[IO<T>::E];
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) {
        p[e] = ok ? phi(x[e]) : 0.f;
        qf.put(c + e, r, p[e]);
      }
      qt.template putrow<IO<T>::E>(r, c, p);
    });
    bk.for_each(nv, [&](int r, int c, const float* x, bool ok) {
      float p[IO<T>::E];
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) {
        p[e] = ok ? phi(x[e]) : 0.f;
        kf.put(c + e, r, p[e]);
      }
      kt.template putrow<IO<T>::E>(r, c, p);
    });
    bv.for_each(nv, [&](int r, int c, const float* x, bool) { vt.template putrow<IO<T>::E>(r, c, x); });
    bd.for_each(nv, [&](int r, int c, const float* x, bool) { ot.template putrow<IO<T>::E>(r, c, x); });
    if (tid < CB) {  // rows past the end keep den = 1, c = 0; valid rows are set below
      sDen[tid] = 1.f;
      sC[tid] = 0.f;
    }
    if (ci > 0) {
      const int p0 = c0 - CB;
      bq.load(Q + offD + (size_t)p0 * D, CB);
      bk.load(K + offD + (size_t)p0 * D, CB);
      bv.load(V + offM + (size_t)p0 * M, CB);
      bd.load(dO + offM + (size_t)p0 * M, CB);
    }
    __syncthreads();

    // ---- S before this chunk
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
      if (ci == 0) {
        const float4 a = *reinterpret_cast<const float4*>(st_start + (16 * db + r16) * M + 16 * mb + 4 * g);
        accS[k] = f32x4_t{a.x, a.y, a.z, a.w};
      } else {
        f32x4_t ds = zero4();
#pragma unroll
        for (int s = 0; s < CB / 32; ++s)
          mmaf<P::dS_a, P::dS_b>(ds, vt.template frag_col<P::dS_a>(16 * mb + r16, 32 * s, g),
                                 kf.template frag<P::dS_b>(16 * db + r16, 32 * s, g));
        accS[k] -= ds;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sp.put(16 * db + r16, 16 * mb + 4 * g + r, accS[k][r]);
    }
    for (int d = l; d < D; d += 64) {
      float zs = 0.f;
      if (16 * w < CB) {
#pragma unroll
        for (int j = 0; j < 16; ++j) zs += kf.get(d, 16 * w + j);
      }
      zpart[w][d] = zs;
    }
    __syncthreads();
    if (tid < D) {
      zcur = ci == 0 ? st_start[D * M + tid] : zcur - (zpart[0][tid] + zpart[1][tid] + zpart[2][tid] + zpart[3][tid]);
      sZ[tid] = zcur;
    }
    __syncthreads();

    // ---- dQ for query rows 16 qrb + r16
    if (has_q) {
      const int ib = qrb, il = 16 * ib + r16;
      constexpr int NO = cmax(P::Bt, P::U1_b);
      Frag<NO> dof[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) dof[s] = ot.template frag<NO>(il, 32 * s, g);
      Frag<P::U2> btf[NPAIR];
      Frag<1> onef[NPAIR];
#pragma unroll
      for (int p = 0; p < NPAIR; ++p) {
        f32x4_t bt[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int jb = 2 * p + h;
          f32x4_t a = zero4();
          if (jb <= ib) {
#pragma unroll
            for (int s = 0; s < M / 32; ++s)
              mmaf<P::Bt, P::Bt>(a, vt.template frag<P::Bt>(16 * jb + r16, 32 * s, g), dof[s]);
            if (jb == ib) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > r16) a[r] = 0.f;  // V_j . dO_i with j > i is masked
            }
          }
          bt[h] = a;
        }
        btf[p] = acc2frag<P::U2>(bt[0], bt[1]);
        bool on[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) on[e] = 32 * p + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4)) <= il;
        onef[p] = mask_frag(on);
      }
      f32x4_t U[DB], ZC[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4_t u = zero4(), zc = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::U1_a, P::U1_b>(u, sp.template frag<P::U1_a>(16 * db + r16, 32 * s, g), dof[s]);
#pragma unroll
        for (int p = 0; p < NPAIR; ++p) {
          if (2 * p <= ib) {
            constexpr int NK = cmax(P::U2, P::Zc);
            const Frag<NK> kfr = kf.template frag_acc<NK>(16 * db + r16, 32 * p, g);
            mmaf<P::U2, P::U2>(u, kfr, btf[p]);
            mmaf<P::Zc, 1>(zc, kfr, onef[p]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) zc[r] += sZ[16 * db + 4 * g + r];
        U[db] = u;    // S_i dO_i
        ZC[db] = zc;  // Z_i
      }
      float pu = 0.f, pz = 0.f;
      float qv[DB][4];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        qt.get4(il, 16 * db + 4 * g, qv[db]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pu += qv[db][r] * U[db][r];
          pz += qv[db][r] * ZC[db][r];
        }
      }
      pu = sum_over_g(pu);  // phi(Q_i)^T S_i dO_i = num_i . dO_i
      pz = sum_over_g(pz);  // phi(Q_i) . Z_i = den_i
      const float invz = 1.f / pz;
      const float odo = pu * invz;  // O_i . dO_i
      if (il < nv) {
        if (g == 0) {
          sC[il] = -odo * invz;
          sDen[il] = pz;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (U[db][r] - ZC[db][r] * odo) * invz * dphi_from_phi(qv[db][r]);
          IO<T>::store4(dQ + offD + (size_t)(c0 + il) * D + 16 * db + 4 * g, o);
        }
      }
      // g_i = dO_i / den_i, feature-major, for this row's quarter of the features
#pragma unroll
      for (int mm = 0; mm < M / 4; mm += 4) {
        float dv[4];
        ot.get4(il, g * (M / 4) + mm, dv);
#pragma unroll
        for (int q = 0; q < 4; ++q) gf.put(g * (M / 4) + mm + q, il, il < nv ? dv[q] * invz : 0.f);
      }
    }
    __syncthreads();

    // ---- reverse-state increment of this chunk (applied after the chunk)
    //      R^T += g^T phi(Q),  r += sum_i c_i phi(Q_i)
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CB / 32; ++s)
        mmaf<P::dR, P::dR>(accR[k], gf.template frag<P::dR>(16 * mb + r16, 32 * s, g),
                           qf.template frag<P::dR>(16 * db + r16, 32 * s, g));
    }
    for (int d = l; d < D; d += 64) {
      float s_ = 0.f;
      if (16 * w < CB) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s_ += sC[16 * w + i] * qf.get(d, 16 * w + i);
      }
      zpart[w][d] = s_;
    }

    // ---- dK, dV for key rows 16 kvrb + r16
    if (has_kv) {
      const int jb = kvrb, jl = 16 * jb + r16;
      constexpr int NKT = cmax(P::At, P::VR);
      Frag<NKT> kfr[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kfr[s] = kt.template frag<NKT>(jl, 32 * s, g);
      constexpr int NVT = cmax(P::Wt, P::KR_b);
      Frag<NVT> vfr[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) vfr[s] = vt.template frag<NVT>(jl, 32 * s, g);
      Frag<P::dK> wfr[NPAIR];
      Frag<P::dV> afr[NPAIR];
#pragma unroll
      for (int p = 0; p < NPAIR; ++p) {
        f32x4_t at[2], wt[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ib = 2 * p + h;
          f32x4_t a = zero4(), b = zero4();
          if (ib >= jb) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
              mmaf<P::At, P::At>(a, qt.template frag<P::At>(16 * ib + r16, 32 * s, g), kfr[s]);
#pragma unroll
            for (int s = 0; s < M / 32; ++s)
              mmaf<P::Wt, P::Wt>(b, ot.template frag<P::Wt>(16 * ib + r16, 32 * s, g), vfr[s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 16 * ib + 4 * g + r;
              b[r] = b[r] / sDen[i] + sC[i];  // g_i . V_j + c_i
              if (ib == jb && 4 * g + r < r16) {
                a[r] = 0.f;
                b[r] = 0.f;
              }
            }
          }
          at[h] = a;
          wt[h] = b;
        }
        wfr[p] = acc2frag<P::dK>(wt[0], wt[1]);
        afr[p] = acc2frag<P::dV>(at[0], at[1]);
      }
      const bool row_ok = jl < nv;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < NPAIR; ++p)
          if (2 * p + 1 >= jb) mmaf<P::dK, P::dK>(acc, qf.template frag_acc<P::dK>(16 * db + r16, 32 * p, g), wfr[p]);
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::KR_a, P::KR_b>(acc, rp.template frag<P::KR_a>(16 * db + r16, 32 * s, g), vfr[s]);
        if (row_ok) {
          float kv[4], o[4];
          kt.get4(jl, 16 * db + 4 * g, kv);
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (acc[r] + sr[16 * db + 4 * g + r]) * dphi_from_phi(kv[r]);
          IO<T>::store4(dK + offD + (size_t)(c0 + jl) * D + 16 * db + 4 * g, o);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < NPAIR; ++p)
          if (2 * p + 1 >= jb) mmaf<P::dV, P::dV>(acc, gf.template frag_acc<P::dV>(16 * mb + r16, 32 * p, g), afr[p]);
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
          mmaf<P::VR, P::VR>(acc, rp.template frag_col<P::VR>(16 * mb + r16, 32 * s, g), kfr[s]);
        if (row_ok) {
          float o[4] = {acc[0], acc[1], acc[2], acc[3]};
          IO<T>::store4(dV + offM + (size_t)(c0 + jl) * M + 16 * mb + 4 * g, o);
        }
      }
    }
    __syncthreads();
    // ---- R for the next (earlier) chunk
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int r = 0; r < 4; ++r) rp.put(16 * db + r16, 16 * mb + 4 * g + r, accR[k][r]);
    }
    if (tid < D) {
      rcur += zpart[0][tid] + zpart[1][tid] + zpart[2][tid] + zpart[3][tid];
      sr[tid] = rcur;
    }
  }
}

// ================================================================= decode
// One RNN step per head (eq. 18-20): S += phi(k) v^T, Z += phi(k),
// y = phi(q)^T S / phi(q)^T Z.  One wavefront per head streams the head's
// D x M float32 state through registers in 1 KiB coalesced rows per
// instruction, updates it in place and reduces phi(q)^T S across lanes.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_decode(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, float* __restrict__ S,
                                                float* __restrict__ Z, T* __restrict__ y, int BH) {
  constexpr int NV = D * M / 4 / 64;  // float4 per lane
  constexpr int CPL = M / 4;          // lanes covering one state row
  constexpr int RPI = 64 / CPL;       // state rows per instruction
  __shared__ float sq[4][D], sk[4][D], sv[4][M];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int head = blockIdx.x * 4 + w;
  const bool live = head < BH;  // a wavefront past the last head only joins the barrier
  auto ld = [](const T* p) -> float {
    if constexpr (sizeof(T) == 4)
      return *reinterpret_cast<const float*>(p);
    else
      return bf2f(*reinterpret_cast<const bf16_t*>(p));
  };
  float zn = 0.f;
  if (live) {
    if (l < D) {
      sq[w][l] = phi(ld(q + (size_t)head * D + l));
      const float pk = phi(ld(k + (size_t)head * D + l));
      sk[w][l] = pk;
      zn = Z[(size_t)head * D + l] + pk;
    }
    if (l < M) sv[w][l] = ld(v + (size_t)head * M + l);
  }
  __syncthreads();
  if (!live) return;

  float4* S4 = reinterpret_cast<float4*>(S + (size_t)head * D * M);
  float4 st[NV];
#pragma unroll
  for (int it = 0; it < NV; ++it) st[it] = S4[l + 64 * it];
  const int m0 = 4 * (l % CPL);
  const float v0 = sv[w][m0], v1 = sv[w][m0 + 1], v2 = sv[w][m0 + 2], v3 = sv[w][m0 + 3];
  float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    const int d = l / CPL + RPI * it;
    const float pk = sk[w][d], pq = sq[w][d];
    float4 s = st[it];
    s.x += pk * v0;
    s.y += pk * v1;
    s.z += pk * v2;
    s.w += pk * v3;
    S4[l + 64 * it] = s;
    y0 += pq * s.x;
    y1 += pq * s.y;
    y2 += pq * s.z;
    y3 += pq * s.w;
  }
#pragma unroll
  for (int off = CPL; off < 64; off <<= 1) {
    y0 += __shfl_xor(y0, off);
    y1 += __shfl_xor(y1, off);
    y2 += __shfl_xor(y2, off);
    y3 += __shfl_xor(y3, off);
  }
  float dn = (l < D) ? sq[w][l] * zn : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dn += __shfl_xor(dn, off);
  if (l < D) Z[(size_t)head * D + l] = zn;
  if (l < CPL) {
    const float inv = 1.f / dn;
    float o[4] = {y0 * inv, y1 * inv, y2 * inv, y3 * inv};
    IO<T>::store4(y + (size_t)head * M + m0, o);
  }
}

}  // namespace la
