// la_kernels.hip -- gfx950 kernels for causal linear attention, phi = elu + 1.
//
// Method: "Transformers are RNNs: Fast Autoregressive Transformers with Linear
// Attention -- part 2/3", eq. 7-20; non-causal form: reading notes on the same
// paper, section 3.2 eq. 5-6; chunked evaluation of the causal sums:
// "Linear Attention/zh", training / parallel form (cut the sequence into
// blocks, quadratic masked attention inside a block, linear state updates
// between blocks).
//
// Work decomposition.  Each (batch*head) sequence is cut into segments of L
// tokens (a multiple of the 64-token chunk); one workgroup of four wavefronts
// owns one (head, segment) and walks its chunks in order, carrying the state
// (S, Z) -- or, in the backward, also the reverse state (R, r) -- in registers
// and LDS.  Segment boundary states come from a per-segment aggregate pass and
// a scan over segments, so all segments run in parallel.
//
// Inside a chunk every contraction is a 16x16 MFMA tile product (fragment
// conventions in la_device.h); wave w owns the 16 query rows 16w..16w+15.
#include "la_device.h"

namespace la {

template <typename T>
struct Lds {
  using type = float;  // float32 storage for float32 I/O
};
template <>
struct Lds<bf16_t> {
  using type = bf16_t;  // operands that are exact or used once-rounded
};

// Per-product precision policies.  Float32 I/O: every product in float32 MFMA.
// bf16 I/O: operands that are exact in bf16 (inputs V, dO, a ones mask) are
// fed as is; computed float32 operands are rounded once where the result only
// needs bf16 accuracy, and split into hi + lo where a later subtraction
// cancels (the query gradient) or where a state accumulates over many tokens.
template <typename T>
struct Policy {
  static constexpr int A_F = P_F32, AV = P_F32, QS = P_F32, S = P_F32, R = P_F32, B = P_F32, U1 = P_F32,
                       U2 = P_F32, Z = P_F32, A = P_F32, K = P_F32, KR = P_F32, V = P_F32, VR = P_F32;
};
template <>
struct Policy<bf16_t> {
  // forward: A = phi(K)phi(Q)^T, AV = V^T A^T, QS = S^T phi(Q)^T, S = V^T phi(K)
  static constexpr int A_F = P_B1, AV = P_B1, QS = P_B1, S = P_B2B;
  // backward: R = dO^T (phi(Q)/den), B = dO.V (exact), U1 = S dO, U2 = phi(K)^T B^T,
  // Z = phi(K)^T 1, A = phi(Q).phi(K), K = phi(Q)^T W, KR = R V, V = dO^T A', VR = R^T phi(K)
  static constexpr int R = P_B2B, B = P_B1, U1 = P_B2A, U2 = P_B3, Z = P_B2A, A = P_B3, K = P_B3, KR = P_B2A,
                       V = P_B2B, VR = P_B3;
};

template <typename T>
constexpr int pad_of() {
  return 16 / (int)sizeof(T);  // keeps every LDS row 16-byte aligned
}

// ===================================================================== F1
// Segment aggregates: agg[bh][seg] = ( sum_j phi(K_j) V_j^T  [D][M],
//                                      sum_j phi(K_j)        [D] )
// over the segment's tokens (eq. 10-11 restricted to one segment).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_seg_state(const T* __restrict__ K, const T* __restrict__ V,
                                                   float* __restrict__ agg, int N, int L, int nseg) {
  using LT = typename Lds<T>::type;
  using Pl = Policy<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  constexpr int PL = pad_of<LT>();
  __shared__ float sKt[D][CH + 4];
  __shared__ LT sVt[M][CH + PL];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;

  f32x4_t acc[NTW];
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();
  float z = 0.f;

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    for_rows<T, D>(Kh + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) sKt[c + e][r] = ok ? phi(x[e]) : 0.f;
    });
    for_rows<T, M>(Vh + (size_t)c0 * M, nv, [&](int r, int c, const float* x, bool) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) lds_put(&sVt[c + e][r], x[e]);
    });
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s)
        mma<Pl::S>(acc[k], frag_std(&sVt[16 * mb + r16][0], 32 * s, g), frag_std(&sKt[16 * db + r16][0], 32 * s, g));
    }
    if (tid < D) {
#pragma unroll 8
      for (int j = 0; j < CH; ++j) z += sKt[tid][j];
    }
    __syncthreads();
  }
  float* out = agg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    // acc[r] = S^T[16mb + 4g + r][16db + r16] = S[d][m]
    *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
        make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
  if (tid < D) out[D * M + tid] = z;
}

// ===================================================================== F2
// Exclusive scan of segment aggregates along the sequence, one thread per
// state element.  ckpt[bh][s] = init + sum_{t<s} agg[bh][t] for s = 0..nseg
// (entry nseg is the final state).  The final state also goes to S_out/Z_out
// and, for the non-causal form, to `total`.
template <int D, int M>
__global__ __launch_bounds__(NT) void k_scan_fwd(const float* __restrict__ agg, const float* __restrict__ S0,
                                                  const float* __restrict__ Z0, float* __restrict__ ckpt,
                                                  float* __restrict__ S_out, float* __restrict__ Z_out,
                                                  float* __restrict__ total, int nseg) {
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
    if (ckpt) ckpt[((size_t)bh * (nseg + 1) + s) * SV + e] = run;
    run += agg[((size_t)bh * nseg + s) * SV + e];
  }
  if (ckpt) ckpt[((size_t)bh * (nseg + 1) + nseg) * SV + e] = run;
  if (S_out) {
    if (e < D * M)
      S_out[(size_t)bh * D * M + e] = run;
    else
      Z_out[(size_t)bh * D + (e - D * M)] = run;
  }
  if (total) total[(size_t)bh * SV + e] = run;
}

// Exclusive reverse scan: rck[bh][s] = sum_{t>s} ragg[bh][t].
template <int D, int M>
__global__ __launch_bounds__(NT) void k_scan_rev(const float* __restrict__ ragg, float* __restrict__ rck, int nseg) {
  constexpr int SV = D * M + D;
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NT + threadIdx.x;
  if (e >= SV) return;
  float run = 0.f;
  for (int s = nseg - 1; s >= 0; --s) {
    rck[((size_t)bh * nseg + s) * SV + e] = run;
    run += ragg[((size_t)bh * nseg + s) * SV + e];
  }
}

// ===================================================================== F3
// Chunked forward over one segment.
//   causal: for each chunk, A^T = phi(K) phi(Q)^T masked to j <= i (eq. 8),
//     num^T = V^T A^T + S^T phi(Q)^T, den = rowsum(A) + phi(Q).Z, O = num/den
//     (eq. 9-12), then S += phi(K)^T V, Z += colsum phi(K) (eq. 10-11).
//   non-causal: num^T = S^T phi(Q)^T with the whole-sequence S, Z (eq. 5-6).
// The start state is read from (Sst, Zst) at element offsets
// bh*sbh + seg*sseg (NULL = zero state).
template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_fwd(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, T* __restrict__ O, float* __restrict__ den_out,
                                             const float* __restrict__ Sst, const float* __restrict__ Zst, long sbh,
                                             long sseg, long zbh, long zseg, float* __restrict__ S_out,
                                             float* __restrict__ Z_out, int N, int L, int nseg) {
  using LT = typename Lds<T>::type;
  using Pl = Policy<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4;
  constexpr int PL = pad_of<LT>();
  constexpr int KC = CAUSAL ? CH : 1;  // causal-only buffers shrink to one column otherwise
  __shared__ float sQ[CH][D + 4];
  __shared__ float sK[KC][D + 4];
  __shared__ float sKt[CAUSAL ? D : 1][KC + 4];
  __shared__ LT sVt[CAUSAL ? M : 1][KC + PL];
  __shared__ float sS[M][D + 4];  // S^T
  __shared__ float sZ[D];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;
  T* Oh = O + (size_t)bh * N * M;

  f32x4_t accS[NTW];
  const float* s_in = Sst ? Sst + bh * sbh + seg * sseg : nullptr;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    if (s_in) {
      const float4 a = *reinterpret_cast<const float4*>(s_in + (16 * db + r16) * M + 16 * mb + 4 * g);
      accS[k] = f32x4_t{a.x, a.y, a.z, a.w};
    } else {
      accS[k] = zero4();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sS[16 * mb + 4 * g + r][16 * db + r16] = accS[k][r];
  }
  if (tid < D) sZ[tid] = Zst ? Zst[bh * zbh + seg * zseg + tid] : 0.f;

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    for_rows<T, D>(Qh + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
      float p[IO<T>::E];
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) p[e] = ok ? phi(x[e]) : 0.f;
      lds_putE<float, IO<T>::E>(&sQ[r][c], p);
    });
    if constexpr (CAUSAL) {
      for_rows<T, D>(Kh + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
        float p[IO<T>::E];
#pragma unroll
        for (int e = 0; e < IO<T>::E; ++e) {
          p[e] = ok ? phi(x[e]) : 0.f;
          sKt[c + e][r] = p[e];
        }
        lds_putE<float, IO<T>::E>(&sK[r][c], p);
      });
      for_rows<T, M>(Vh + (size_t)c0 * M, nv, [&](int r, int c, const float* x, bool) {
#pragma unroll
        for (int e = 0; e < IO<T>::E; ++e) lds_put(&sVt[c + e][r], x[e]);
      });
    }
    __syncthreads();

    F8 qf[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = frag_std(&sQ[16 * w + r16][0], 32 * s, g);

    float dp = 0.f;
    f32x4_t accA[4];
    if constexpr (CAUSAL) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) mma<Pl::A_F>(a, frag_std(&sK[16 * jb + r16][0], 32 * s, g), qf[s]);
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
    }
#pragma unroll
    for (int dd = 0; dd < D / 4; ++dd) dp += sQ[16 * w + r16][g * (D / 4) + dd] * sZ[g * (D / 4) + dd];
    dp = sum_over_g(dp);
    const float inv = 1.f / dp;
    const int il = 16 * w + r16;
    const bool row_ok = il < nv;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t acc = zero4();
      if constexpr (CAUSAL) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p <= w) mma<Pl::AV>(acc, frag_acc(&sVt[16 * mb + r16][0], 32 * p, g), acc2frag(accA[2 * p], accA[2 * p + 1]));
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mma<Pl::QS>(acc, frag_std(&sS[16 * mb + r16][0], 32 * s, g), qf[s]);
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
          mma<Pl::S>(accS[k], frag_std(&sVt[16 * mb + r16][0], 32 * s, g), frag_std(&sKt[16 * db + r16][0], 32 * s, g));
      }
      float zadd = 0.f;
      if (tid < D) {
#pragma unroll 8
        for (int j = 0; j < CH; ++j) zadd += sKt[tid][j];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[16 * mb + 4 * g + r][16 * db + r16] = accS[k][r];
      }
      if (tid < D) sZ[tid] += zadd;
    } else {
      __syncthreads();
    }
  }
  if constexpr (CAUSAL) {
    if (S_out) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
        *reinterpret_cast<float4*>(S_out + (size_t)bh * D * M + (16 * db + r16) * M + 16 * mb + 4 * g) =
            make_float4(accS[k][0], accS[k][1], accS[k][2], accS[k][3]);
      }
      if (tid < D) Z_out[(size_t)bh * D + tid] = sZ[tid];
    }
  }
}

// ------------------------------------------------------------ grad staging
// Stage one chunk of dO (feature-major, exact), den_i and the denominator's
// share c_i = -(dO_i . O_i) / den_i from the stored O and den.  Rows past the
// end get dO = 0, den = 1, c = 0.
template <typename T, int M, typename LT, int PGT>
__device__ __forceinline__ void stage_grad(const T* dOh, const T* Oh, const float* denh, int nv, LT (*sdOt)[PGT],
                                           float* sDen, float* sC) {
  constexpr int E = IO<T>::E;
  constexpr int PR = M / E;
  for_rows<T, M>(dOh, nv, [&](int r, int c, const float* d, bool ok) {
    float o[E];
    float dn = 1.f;
    if (ok) {
      IO<T>::load(Oh + (size_t)r * M + c, o);
      dn = denh[r];
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = 0.f;
    }
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part += d[e] * o[e];
#pragma unroll
    for (int off = PR / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off);
#pragma unroll
    for (int e = 0; e < E; ++e) lds_put(&sdOt[c + e][r], d[e]);
    if (c == 0) {
      sDen[r] = dn;
      sC[r] = -part / dn;
    }
  });
}

// ===================================================================== B1
// Segment aggregates of the reverse state: ragg[bh][seg] =
//   ( R = sum_i phi(Q_i) g_i^T [D][M],  r = sum_i c_i phi(Q_i) [D] )
// i.e. the backward-running sums of eq. 14-15 over one segment, with the
// upstream [g, c] of the numerator and the denominator (g_i = dO_i / den_i),
// taken from the forward's O and den.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_seg_rstate(const T* __restrict__ Q, const T* __restrict__ O,
                                                    const float* __restrict__ den, const T* __restrict__ dO,
                                                    float* __restrict__ ragg, int N, int L, int nseg) {
  using LT = typename Lds<T>::type;
  using Pl = Policy<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  constexpr int PL = pad_of<LT>();
  __shared__ float sQt[D][CH + 4];
  __shared__ LT sdOt[M][CH + PL];
  __shared__ float sDen[CH], sC[CH];

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

  for (int c0 = t0; c0 < t1; c0 += CH) {
    const int nv = min(CH, t1 - c0);
    for_rows<T, D>(Qh + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) sQt[c + e][r] = ok ? phi(x[e]) : 0.f;
    });
    stage_grad<T, M, LT, CH + PL>(dOh + (size_t)c0 * M, Oh + (size_t)c0 * M, denh + c0, nv, sdOt, sDen, sC);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        F8 b = frag_std(&sQt[16 * db + r16][0], 32 * s, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) b.v[e] /= sDen[32 * s + 8 * g + e];
        mma<Pl::R>(acc[k], frag_std(&sdOt[16 * mb + r16][0], 32 * s, g), b);
      }
    }
    if (tid < D) {
#pragma unroll 8
      for (int i = 0; i < CH; ++i) rr += sC[i] * sQt[tid][i];
    }
    __syncthreads();
  }
  float* out = ragg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
        make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
  if (tid < D) out[D * M + tid] = rr;
}

// ===================================================================== B3
// Backward over one segment, chunks in reverse order.  Registers carry
//   S (forward sum of phi(K) V^T, eq. 13), walked backwards from the
//     segment's end state by removing each chunk's contribution (the first
//     chunk restarts from the segment's start state), and
//   R (backward sum of phi(Q) g^T, eq. 14-15) from the segment's suffix.
// Per chunk, wave w produces
//   dQ for rows 16w..: with u_i = S_i dO_i, Z_i the inclusive normaliser,
//     den_i = phi(Q_i).Z_i and O_i.dO_i = phi(Q_i).u_i / den_i (both
//     recomputed here in float32),
//     dphiQ_i = (u_i - Z_i (O_i.dO_i)) / den_i
//     which is eq. 13's S_i g_i plus the denominator's share c_i Z_i, with
//     g_i = dO_i / den_i and c_i = -(O_i.dO_i) / den_i;
//   dK, dV for rows 16w..: dphiK_j = sum_{i>=j} phi(Q_i)(g_i.V_j + c_i)
//     + R V_j + r, dV_j = sum_{i>=j} g_i (phi(Q_i).phi(K_j)) + R^T phi(K_j)
//     (eq. 14-15 on [V, 1] with upstream [g, c]);
// and the chain rule through phi.  The stored O and den are not read: the
// recomputed den_i and O_i.dO_i are exact to float32, so g_i.V_j + c_i
// cancels exactly where V_j = O_i even for bf16 storage.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_bwd(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, const T* __restrict__ dO,
                                             const float* __restrict__ ckpt, const float* __restrict__ rck,
                                             T* __restrict__ dQ, T* __restrict__ dK, T* __restrict__ dV, int N, int L,
                                             int nseg) {
  using LT = typename Lds<T>::type;
  using Pl = Policy<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  constexpr int PL = pad_of<LT>();
  __shared__ float sQt[D][CH + 4];  // phi(Q), feature-major
  __shared__ float sKt[D][CH + 4];  // phi(K), feature-major
  __shared__ float sK[CH][D + 4];   // phi(K), token-major
  __shared__ LT sV[CH][M + PL];     // V, token-major (exact)
  __shared__ LT sdO[CH][M + PL];    // dO, token-major (exact)
  __shared__ LT sdOt[M][CH + PL];   // dO, feature-major (exact)
  __shared__ float sR[D][M + 4];    // R for this chunk, [d][m]
  __shared__ float sS[D][M + 4];    // S before this chunk, [d][m]
  __shared__ float sZ[D], sr[D], sDen[CH], sC[CH];

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;

  const float* st_start = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
  const float* st_end = st_start + SV;
  const float* rst = rck ? rck + ((size_t)bh * nseg + seg) * SV : nullptr;

  f32x4_t accS[NTW], accR[NTW];  // S^T and R^T tiles: [16mb + 4g + r][16db + r16]
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    const float4 a = *reinterpret_cast<const float4*>(st_end + (16 * db + r16) * M + 16 * mb + 4 * g);
    accS[k] = f32x4_t{a.x, a.y, a.z, a.w};
    if (rst) {
      const float4 b = *reinterpret_cast<const float4*>(rst + (16 * db + r16) * M + 16 * mb + 4 * g);
      accR[k] = f32x4_t{b.x, b.y, b.z, b.w};
    } else {
      accR[k] = zero4();
    }
    float rv[4] = {accR[k][0], accR[k][1], accR[k][2], accR[k][3]};
    lds_put4(&sR[16 * db + r16][16 * mb + 4 * g], rv);
  }
  float zcur = 0.f, rcur = 0.f;
  if (tid < D) {
    zcur = st_end[D * M + tid];
    rcur = rst ? rst[D * M + tid] : 0.f;
    sr[tid] = rcur;
  }

  const int nchunk = (t1 - t0 + CH - 1) / CH;
  for (int ci = nchunk - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * CH;
    const int nv = min(CH, t1 - c0);
    // ---- stage
    for_rows<T, D>(Q + offD + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) sQt[c + e][r] = ok ? phi(x[e]) : 0.f;
    });
    for_rows<T, D>(K + offD + (size_t)c0 * D, nv, [&](int r, int c, const float* x, bool ok) {
      float p[IO<T>::E];
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) {
        p[e] = ok ? phi(x[e]) : 0.f;
        sKt[c + e][r] = p[e];
      }
      lds_putE<float, IO<T>::E>(&sK[r][c], p);
    });
    for_rows<T, M>(V + offM + (size_t)c0 * M, nv, [&](int r, int c, const float* x, bool) {
      lds_putE<LT, IO<T>::E>(&sV[r][c], x);
    });
    for_rows<T, M>(dO + offM + (size_t)c0 * M, nv, [&](int r, int c, const float* x, bool) {
      lds_putE<LT, IO<T>::E>(&sdO[r][c], x);
#pragma unroll
      for (int e = 0; e < IO<T>::E; ++e) lds_put(&sdOt[c + e][r], x[e]);
    });
    if (tid < CH) {  // rows past the end keep den = 1, c = 0; valid rows are set below
      sDen[tid] = 1.f;
      sC[tid] = 0.f;
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
        for (int s = 0; s < CH / 32; ++s)
          mma<Pl::S>(ds, frag_col(&sV[0][16 * mb + r16], M + PL, 32 * s, g), frag_std(&sKt[16 * db + r16][0], 32 * s, g));
        accS[k] -= ds;
      }
      float sv[4] = {accS[k][0], accS[k][1], accS[k][2], accS[k][3]};
      lds_put4(&sS[16 * db + r16][16 * mb + 4 * g], sv);
    }
    if (tid < D) {
      if (ci == 0) {
        zcur = st_start[D * M + tid];
      } else {
        float zs = 0.f;
#pragma unroll 8
        for (int j = 0; j < CH; ++j) zs += sKt[tid][j];
        zcur -= zs;
      }
      sZ[tid] = zcur;
    }
    __syncthreads();

    // ---- dQ for query rows 16w + r16
    {
      const int il = 16 * w + r16;
      f32x4_t Bt[4];  // Bt[jb][r] = V_j . dO_i, j = 16jb + 4g + r, masked to j <= i
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mma<Pl::B>(a, frag_std(&sV[16 * jb + r16][0], 32 * s, g), frag_std(&sdO[il][0], 32 * s, g));
          if (jb == w) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (4 * g + r > r16) a[r] = 0.f;
          }
        }
        Bt[jb] = a;
      }
      f32x4_t U[DB], ZC[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4_t u = zero4(), zc = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mma<Pl::U1>(u, frag_std(&sS[16 * db + r16][0], 32 * s, g), frag_std(&sdO[il][0], 32 * s, g));
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if (2 * p <= w) {
            const F8 kf = frag_acc(&sKt[16 * db + r16][0], 32 * p, g);
            mma<Pl::U2>(u, kf, acc2frag(Bt[2 * p], Bt[2 * p + 1]));
            F8 ones;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = 32 * p + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
              ones.v[e] = (j <= il) ? 1.f : 0.f;
            }
            mma<Pl::Z>(zc, kf, ones);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) zc[r] += sZ[16 * db + 4 * g + r];
        U[db] = u;    // S_i dO_i
        ZC[db] = zc;  // Z_i
      }
      float pu = 0.f, pz = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ph = sQt[16 * db + 4 * g + r][il];
          pu += ph * U[db][r];
          pz += ph * ZC[db][r];
        }
      pu = sum_over_g(pu);  // phi(Q_i)^T S_i dO_i = num_i . dO_i
      pz = sum_over_g(pz);  // phi(Q_i) . Z_i = den_i
      const float invz = 1.f / pz;
      const float odo = pu * invz;  // O_i . dO_i
      if (g == 0 && il < nv) {
        sC[il] = -odo * invz;
        sDen[il] = pz;
      }
      if (il < nv) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ph = sQt[16 * db + 4 * g + r][il];
            o[r] = (U[db][r] - ZC[db][r] * odo) * invz * dphi_from_phi(ph);
          }
          IO<T>::store4(dQ + offD + (size_t)(c0 + il) * D + 16 * db + 4 * g, o);
        }
      }
    }
    __syncthreads();

    // ---- reverse-state increment of this chunk (applied after the chunk)
    //      R^T += dO^T (phi(Q) / den),  r += sum_i c_i phi(Q_i)
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        F8 b = frag_std(&sQt[16 * db + r16][0], 32 * s, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) b.v[e] /= sDen[32 * s + 8 * g + e];
        mma<Pl::R>(accR[k], frag_std(&sdOt[16 * mb + r16][0], 32 * s, g), b);
      }
    }
    float rnext = 0.f;
    if (tid < D) {
      float rs = 0.f;
#pragma unroll 8
      for (int i = 0; i < CH; ++i) rs += sC[i] * sQt[tid][i];
      rnext = rcur + rs;
    }

    // ---- dK, dV for key rows 16w + r16
    {
      const int jl = 16 * w + r16;
      f32x4_t At[4], Wt[4];  // [ib][r]: row i = 16ib + 4g + r, column j = jl; masked to i >= j
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4_t a = zero4(), b = zero4();
        if (ib >= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s)
            mma<Pl::A>(a, frag_col(&sQt[0][16 * ib + r16], CH + 4, 32 * s, g), frag_std(&sK[jl][0], 32 * s, g));
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mma<Pl::B>(b, frag_std(&sdO[16 * ib + r16][0], 32 * s, g), frag_std(&sV[jl][0], 32 * s, g));
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * g + r;
            const float inv = 1.f / sDen[i];
            a[r] *= inv;                // phi(Q_i).phi(K_j) / den_i
            b[r] = b[r] * inv + sC[i];  // g_i . V_j + c_i
            if (ib == w && 4 * g + r < r16) {
              a[r] = 0.f;
              b[r] = 0.f;
            }
          }
        }
        At[ib] = a;
        Wt[ib] = b;
      }
      const bool row_ok = jl < nv;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p + 1 >= w) mma<Pl::K>(acc, frag_acc(&sQt[16 * db + r16][0], 32 * p, g), acc2frag(Wt[2 * p], Wt[2 * p + 1]));
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mma<Pl::KR>(acc, frag_std(&sR[16 * db + r16][0], 32 * s, g), frag_std(&sV[jl][0], 32 * s, g));
        if (row_ok) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 16 * db + 4 * g + r;
            o[r] = (acc[r] + sr[d]) * dphi_from_phi(sKt[d][jl]);
          }
          IO<T>::store4(dK + offD + (size_t)(c0 + jl) * D + 16 * db + 4 * g, o);
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p + 1 >= w) mma<Pl::V>(acc, frag_acc(&sdOt[16 * mb + r16][0], 32 * p, g), acc2frag(At[2 * p], At[2 * p + 1]));
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
          mma<Pl::VR>(acc, frag_col(&sR[0][16 * mb + r16], M + 4, 32 * s, g), frag_std(&sK[jl][0], 32 * s, g));
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
      float rv[4] = {accR[k][0], accR[k][1], accR[k][2], accR[k][3]};
      lds_put4(&sR[16 * db + r16][16 * mb + 4 * g], rv);
    }
    if (tid < D) {
      rcur = rnext;
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
