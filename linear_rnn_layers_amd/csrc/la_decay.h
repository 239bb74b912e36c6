// la_decay.h -- gfx950 kernels for the decayed recurrence.
//
// Method: "Linear Attention/zh", variants and extensions: RetNet replaces the
// unbounded running sum by S_t = gamma S_{t-1} + phi(k_t) v_t^T, gated linear
// attention makes the decay depend on the data.  Here the decay is one
// scalar a_t = exp(logA_t) in (0, 1] per token and head; the normaliser Z
// takes the same decay, so the output stays a weighted average:
//   S_t = a_t S_{t-1} + phi(K_t) V_t^T,  Z_t = a_t Z_{t-1} + phi(K_t),
//   O_t = phi(Q_t)^T S_t / phi(Q_t)^T Z_t.
// Token j's weight at query i >= j is exp(L_i - L_j) with L the running sum
// of logA.  In a 64-token chunk with lam the chunk-local inclusive running
// sum of logA:
//   S_i = exp(lam_i) S_before + sum_{j <= i} exp(lam_i - lam_j) phi(K_j) V_j^T
//   S_after = exp(lam_last) S_before + sum_j exp(lam_last - lam_j) phi(K_j) V_j^T
// Every exponent is <= 0, so no factor overflows; the factors multiply the
// intra-chunk attention tiles elementwise, scale the state term per query
// row, and scale the token operand of the state update in registers
// (scale_frag), so no decayed copy of an operand is staged.
//
// Backward (reverse-mode through the recurrence, the same quotient rule as
// the plain method on [V, 1] with upstream G_i = [g_i, c_i]):
//   dphiQ_i = S_i G_i                    (forward order: pass k_dbq)
//   R_j = sum_{i >= j} exp(L_i - L_j) phi(Q_i) G_i^T + exp(L_N - L_j) [dS_N | dZ_N]
//   dphiK_j = R_j [V_j, 1],  dV_j = R_j^T phi(K_j)   (reverse order: k_dbkv)
//   dlogA_l = sum_{m >= l} (phi(Q_m).dphiQ_m - phi(K_m).dphiK_m) + <[dS_N|dZ_N], [S_N|Z_N]>
// (logA_l enters every weight exp(L_i - L_j) with j < l <= i and the final
// state).  O_m is a ratio of two linear functions of phi(Q_m), homogeneous
// of degree 0, so phi(Q_m).dphiQ_m = 0 exactly and only the key terms are
// summed (k_dbkv within each segment, k_dla_fix across segments).  The query side needs S_i, which
// only the forward order reaches stably (subtracting later tokens from the
// state after a chunk would multiply by exp(+lam)); the key side runs in
// reverse, where the carried R only decays.
#pragma once

#include "la_kernels.h"

namespace la {

// Planes per staged operand of the decayed backward (the products use the
// same counts on both sides): float32 I/O keeps float32 level throughout;
// bf16 I/O keeps phi(Q), phi(K) and the carried states in two planes (inputs
// V and dO are exact in one).
template <typename T>
struct DPrec;
template <>
struct DPrec<bf16_t> {
  static constexpr int Q = 2, K = 2, V = 1, DO = 1, S = 2, G = 2, R = 2, W = 2;
  // the key pass's dV side: the weighted attention tile (phi(Q).phi(K), then
  // as the operand of dO A) and phi(K) in R+^T phi(K) -- per-term products
  // that cancel nothing -- take one plane (R+ keeps R)
  static constexpr int Av = 1, Wv = 1, Kv = 1;
};
template <>
struct DPrec<float> {
  static constexpr int Q = 3, K = 3, V = 3, DO = 3, S = 3, G = 2, R = 3, W = 3;
  static constexpr int Av = 3, Wv = 3, Kv = 3;
};

__device__ __forceinline__ float exp_nat(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Inclusive running sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_incl_sum(float x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}

// A fragment (standard map, k = 8g + e) whose k-th slice is multiplied by
// f[e]: the planes are summed, scaled and split again.
template <int N>
__device__ __forceinline__ Frag<N> scale_frag(const Frag<N>& a, const float* f) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = 0.f;
#pragma unroll
    for (int p = N - 1; p >= 0; --p) x += (float)a.p[p][e];
    v[e] = x * f[e];
  }
  return split8<N>(v);
}

// logA of the chunk's tokens, one per lane (0 past the end: no decay there).
__device__ __forceinline__ float load_ell(const float* la, int c0, int nv) {
  const int l = threadIdx.x & 63;
  return l < nv ? la[c0 + l] : 0.f;
}

// ------------------------------------------------------------ aggregates
// Decayed segment aggregates: agg[bh][seg] = sum_j exp(L_end - L_j)
// (phi(K_j) V_j^T, phi(K_j)) over the segment (S layout as k_seg_state), and
// dlam[bh][seg] = sum of logA over the segment.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_dseg_state(const T* __restrict__ K, const T* __restrict__ V,
                                                    const float* __restrict__ logA, float* __restrict__ agg,
                                                    float* __restrict__ dlam, int N, int L, int nseg, int fm) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  __shared__ Planes<P::FKF, CH, D> kt;
  __shared__ Planes<P::FV, CH, M> vt;
  __shared__ alignas(16) float sF[CH];  // exp(lam_last - lam_j)

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;
  const float* la = logA + (size_t)bh * N;
  const Frag<1> ones = ones_frag();

  f32x4_t acc[NTW], accZ = zero4();  // S layout; accZ[r] = Z[16db + 4g + r]
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();
  float total = 0.f;

  RowBuf<T, CH, D> bk[2];
  RowBuf<T, CH, M> bv[2];
  float ell[2];
  auto fetch = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      bk[b].load(Kh + (size_t)c0 * D, nv);
      bv[b].load(Vh + (size_t)c0 * M, nv);
      ell[b] = load_ell(la, c0, nv);
    }
  };
  auto chunk = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    const float lam = wave_incl_sum(ell[b]);
    const float last = __shfl(lam, 63, 64);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    bk[b].stage_phi(kt, nv, nullptr, fm);
    bv[b].stage_values(vt);
    if (w == 0) sF[l] = exp_nat(last - lam);
    fetch(b, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    const float dec = exp_nat(last);
#pragma unroll
    for (int k = 0; k < NTW; ++k) acc[k] *= dec;
    accZ *= dec;
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      // A operand phi(K)^T: a[e] = phi(K)[32s + 8g + e][16db + r16], scaled per token
      const Frag<P::FKF> ka =
          scale_frag<P::FKF>(kt.template tfrag<P::FKF>(32 * s, 16 * db, g, r16), &sF[32 * s + 8 * g]);
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int mb = (w + 4 * k) / DB;
        mmaf<P::FKF, P::FV>(acc[k], ka, vt.template tfrag<P::FV>(32 * s, 16 * mb, g, r16));
      }
      if (zw) mmaf<P::FKF, 1>(accZ, ka, ones);
    }
    total += last;
  };
  fetch(0, t0);
  fetch(1, t0 + CH);
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(0, c0);
    if (c0 + CH < t1) chunk(1, c0 + CH);
  }
  float* out = agg + ((size_t)bh * nseg + seg) * SV;
  store_S_tiles<D, M, NTW>(out, acc, w, r16, g);
  if (zw && r16 == 0)
    *reinterpret_cast<float4*>(out + D * M + 16 * db + 4 * g) = make_float4(accZ[0], accZ[1], accZ[2], accZ[3]);
  if (tid == 0) dlam[(size_t)bh * nseg + seg] = total;
}

// Decayed prefix states: pref[bh][0] = (S0, Z0) or zero, pref[bh][s + 1] =
// exp(dlam[s]) pref[bh][s] + agg[bh][s].
template <int D, int M>
__global__ __launch_bounds__(NT) void k_dscan_states(const float* __restrict__ agg, const float* __restrict__ dlam,
                                                      const float* __restrict__ S0, const float* __restrict__ Z0,
                                                      float* __restrict__ pref, int nseg) {
  constexpr int SV = D * M + D, BT = 16;
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NT + threadIdx.x;
  if (e >= SV) return;
  float run = 0.f;
  if (e < D * M) {
    if (S0) run = S0[(size_t)bh * D * M + e];
  } else {
    if (Z0) run = Z0[(size_t)bh * D + (e - D * M)];
  }
  const float* a = agg + (size_t)bh * nseg * SV + e;
  const float* dl = dlam + (size_t)bh * nseg;
  float* o = pref + (size_t)bh * (nseg + 1) * SV + e;
  for (int s0 = 0; s0 < nseg; s0 += BT) {
    float v[BT], f[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      v[j] = s0 + j < nseg ? a[(size_t)(s0 + j) * SV] : 0.f;
      f[j] = s0 + j < nseg ? exp_nat(dl[s0 + j]) : 1.f;
    }
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      if (s0 + j < nseg) {
        o[(size_t)(s0 + j) * SV] = run;
        run = f[j] * run + v[j];
      }
    }
  }
  o[(size_t)nseg * SV] = run;
}

// ---------------------------------------------------------------- forward
// Decayed causal forward over one segment (four wavefronts; wave w owns
// tokens 16w..16w+15 of a 64-token chunk).  The start state is entry seg of
// `pref` when given, else (S0, Z0) or zero (one segment); with one segment
// and a checkpoint the start and final states go to its entries 0 and 1.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_dfwd(const T* __restrict__ Q, const T* __restrict__ K,
                                              const T* __restrict__ V, const float* __restrict__ logA,
                                              T* __restrict__ O, float* __restrict__ den_out,
                                              const float* __restrict__ pref, const float* __restrict__ S0,
                                              const float* __restrict__ Z0, float* __restrict__ ckpt,
                                              float* __restrict__ S_out, float* __restrict__ Z_out, int N, int L,
                                              int nseg, int fm) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  __shared__ Planes<P::FQ, CH, D> qt;
  __shared__ Planes<P::FKF, CH, D> kt;
  __shared__ Planes<P::FV, CH, M> vt;
  __shared__ Planes<P::FS, M, D> st;   // S^T
  __shared__ Planes<P::FZ, 16, D> zr;  // 16 copies of Z
  __shared__ alignas(16) float slam[CH];
  __shared__ alignas(16) float sF[CH];

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;
  const float* la = logA + (size_t)bh * N;
  T* Oh = O + (size_t)bh * N * M;
  const Frag<1> ones = ones_frag();

  RowBuf<T, CH, D> bq[2], bk[2];
  RowBuf<T, CH, M> bv[2];
  float ell[2];
  auto fetch = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      bq[b].load(Qh + (size_t)c0 * D, nv);
      bk[b].load(Kh + (size_t)c0 * D, nv);
      bv[b].load(Vh + (size_t)c0 * M, nv);
      ell[b] = load_ell(la, c0, nv);
    }
  };
  fetch(0, t0);
  fetch(1, t0 + CH);

  f32x4_t accS[NTW], accZ = zero4();  // S layout
#pragma unroll
  for (int k = 0; k < NTW; ++k) accS[k] = zero4();
  const float* st0 = pref ? pref + ((size_t)bh * (nseg + 1) + seg) * SV : (S0 ? S0 + (size_t)bh * D * M : nullptr);
  const float* zt0 = pref ? st0 + D * M : (Z0 ? Z0 + (size_t)bh * D : nullptr);
  if (st0) add_S_tiles<D, M, NTW>(accS, st0, 0, 0, 1, w, r16, g);
  if (zw && zt0) {
    const float4 z4 = *reinterpret_cast<const float4*>(zt0 + 16 * db + 4 * g);
    accZ = f32x4_t{z4.x, z4.y, z4.z, z4.w};
  }
  auto write_state = [&](float* dS, float* dZ) {
    store_S_tiles<D, M, NTW>(dS, accS, w, r16, g);
    if (zw && r16 == 0)
      *reinterpret_cast<float4*>(dZ + 16 * db + 4 * g) = make_float4(accZ[0], accZ[1], accZ[2], accZ[3]);
  };
  auto stage_state = [&]() {
    float v4[4];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      acc_to4(accS[k], v4);
      st.put4(16 * ((w + 4 * k) / DB) + r16, 16 * db + 4 * g, v4);
    }
    if (zw) {
      acc_to4(accZ, v4);
      zr.put4(r16, 16 * db + 4 * g, v4);
    }
  };
  if (!pref && ckpt) write_state(ckpt + (size_t)bh * 2 * SV, ckpt + (size_t)bh * 2 * SV + D * M);
  stage_state();

  auto chunk = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    const float lam = wave_incl_sum(ell[b]);
    const float last = __shfl(lam, 63, 64);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    bq[b].stage_phi(qt, nv, nullptr, fm);
    bk[b].stage_phi(kt, nv, nullptr, fm);
    bv[b].stage_values(vt);
    if (w == 0) {
      slam[l] = lam;
      sF[l] = exp_nat(last - lam);
    }
    fetch(b, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);

    const int il = 16 * w + r16;
    const float lam_i = slam[il], e_i = exp_nat(lam_i);
    Frag<P::FQ> qf[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = qt.template frag<P::FQ>(il, 32 * s, g);

    // A^T[j][i] = phi(K_j).phi(Q_i) exp(lam_i - lam_j) for j <= i
    Frag<P::FA> af[2];
    float dp = 0.f;
    {
      f32x4_t accA[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) mmaf<P::FK, P::FQ>(a, kt.template frag<P::FK>(16 * jb + r16, 32 * s, g), qf[s]);
          const float4 lj = *reinterpret_cast<const float4*>(&slam[16 * jb + 4 * g]);
          const float ljv[4] = {lj.x, lj.y, lj.z, lj.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool on = jb < w || 4 * g + r <= r16;
            a[r] = on ? a[r] * exp_nat(lam_i - ljv[r]) : 0.f;
            dp += a[r];
          }
        }
        accA[jb] = a;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) af[p] = acc2frag<P::FA>(accA[2 * p], accA[2 * p + 1]);
      dp = sum_over_g(dp);
    }
    f32x4_t dn = zero4();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) mmaf<P::FZ, P::FQ>(dn, zr.template frag<P::FZ>(r16, 32 * s, g), qf[s]);
    const float den = dp + e_i * dn[0];
    const float inv = 1.f / den;
    const bool row_ok = il < nv;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mmaf<P::FS, P::FQ>(acc, st.template frag<P::FS>(16 * mb + r16, 32 * s, g), qf[s]);
      acc *= e_i;  // the state before the chunk, decayed to token i
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (2 * p <= w) mmaf<P::FV, P::FA>(acc, vt.template tfrag_acc<P::FV>(32 * p, 16 * mb, g, r16), af[p]);
      if (row_ok) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = acc[r] * inv;
        IO<T>::store4(Oh + (size_t)(c0 + il) * M + 16 * mb + 4 * g, o);
      }
    }
    if (den_out && g == 0 && row_ok) den_out[(size_t)bh * N + c0 + il] = den;

    // S_after = exp(lam_last) S_before + sum_j exp(lam_last - lam_j) phi(K_j) V_j^T
    const float dec = exp_nat(last);
#pragma unroll
    for (int k = 0; k < NTW; ++k) accS[k] *= dec;
    accZ *= dec;
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      const Frag<P::FKF> ka =
          scale_frag<P::FKF>(kt.template tfrag<P::FKF>(32 * s, 16 * db, g, r16), &sF[32 * s + 8 * g]);
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int mb = (w + 4 * k) / DB;
        mmaf<P::FKF, P::FV>(accS[k], ka, vt.template tfrag<P::FV>(32 * s, 16 * mb, g, r16));
      }
      if (zw) mmaf<P::FKF, 1>(accZ, ka, ones);
    }
    __syncthreads();
    stage_state();
  };
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(0, c0);
    if (c0 + CH < t1) chunk(1, c0 + CH);
  }
  if (seg == nseg - 1) {
    if (!pref && ckpt) write_state(ckpt + (size_t)bh * 2 * SV + SV, ckpt + (size_t)bh * 2 * SV + SV + D * M);
    if (S_out) write_state(S_out + (size_t)bh * D * M, Z_out + (size_t)bh * D);
  }
}

// ------------------------------------------------------- backward: queries
// Query pass over one segment in forward order, from the segment's start
// state (checkpoint entry seg).  Per chunk, for the wave's query rows i:
//   den_i = sum_{j<=i} A_ij + e_i phi(Q_i).Z,  A_ij = phi(Q_i).phi(K_j) exp(lam_i - lam_j),
//   O_i.dO_i = (sum_j A_ij (dO_i.V_j) + e_i phi(Q_i).(S dO_i)) / den_i,  e_i = exp(lam_i),
//   dphiQ_i = (sum_{j<=i} exp(lam_i - lam_j) (dO_i.V_j - O_i.dO_i) phi(K_j)
//              + e_i (S dO_i - (O_i.dO_i) Z)) / den_i,
// with S, Z the state before the chunk.  Writes dQ, gc[i] = (1/den_i, c_i)
// (c_i = -(O_i.dO_i)/den_i), the segment's reverse
// aggregate ragg = sum_i exp(L_i - L_start) phi(Q_i) [g_i | c_i]^T (S^T
// layout as the causal one; L_start the running sum before the segment) and
// dlam[seg] = sum of logA over the segment.
//
// Eight wavefronts in two roles, one of each per SIMD: wavefronts 0-3 own the
// query rows (dQ, 1/den, c and the weighted [g | c] rows), wavefronts 4-7
// carry the state (its update for the next chunk runs while the query rows
// are worked on) and, after the barrier that publishes [g | c], the reverse
// aggregate.
template <typename T, int D, int M>
__global__ __launch_bounds__(2 * NT) void k_dbq(const T* __restrict__ Q, const T* __restrict__ K,
                                                 const T* __restrict__ V, const T* __restrict__ dO,
                                                 const float* __restrict__ logA, const float* __restrict__ ckpt,
                                                 T* __restrict__ dQ, float2* __restrict__ gc,
                                                 float* __restrict__ ragg, float* __restrict__ dlam, int N, int L,
                                                 int nseg, int fm) {
  using P = DPrec<T>;
  constexpr int NTH = 2 * NT, DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  __shared__ Planes<P::Q, CH, D> qt;
  __shared__ Planes<P::K, CH, D> kt;
  __shared__ Planes<P::V, CH, M> vt;
  __shared__ Planes<P::DO, CH, M> ot;
  __shared__ Planes<P::S, D, M> sp;       // S before the chunk, [d][m]
  __shared__ Planes<P::G, CH, M + 16> gt;  // exp(L_i - L_start) [g_i | c_i | 0]
  __shared__ alignas(16) float sZ[D];
  __shared__ alignas(16) float slam[CH];
  __shared__ alignas(16) float sF[CH];

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const bool qrole = w < 4;
  const int sw = w & 3;  // rank among the state wavefronts
  const int db = sw % DB;
  const bool zw = !qrole && sw < DB;
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;
  const float* la = logA + (size_t)bh * N;
  const Frag<1> ones = ones_frag();
  gt.zero_cols(M + 1, M + 16, NTH);

  constexpr int OD_ = RowBuf<T, CH, D, NTH>::VEC < NTH ? NTH / 2 : 0;
  constexpr int OM_ = RowBuf<T, CH, M, NTH>::VEC < NTH ? NTH / 2 : 0;
  RowBuf<T, CH, D, NTH> bq[2];
  RowBuf<T, CH, D, NTH, OD_> bk[2];
  RowBuf<T, CH, M, NTH> bv[2];
  RowBuf<T, CH, M, NTH, OM_> bd[2];
  float ell[2];
  auto fetch = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      bq[b].load(Q + offD + (size_t)c0 * D, nv);
      bk[b].load(K + offD + (size_t)c0 * D, nv);
      bv[b].load(V + offM + (size_t)c0 * M, nv);
      bd[b].load(dO + offM + (size_t)c0 * M, nv);
      ell[b] = load_ell(la, c0, nv);
    }
  };
  fetch(0, t0);
  fetch(1, t0 + CH);

  // state wavefronts: S^T layout accS[k][r] = S[16db + r16][16mb + 4g + r] (tile sw + 4k),
  // accZ[.] = Z[16db + r16]; the reverse aggregate in the same layout
  f32x4_t accS[NTW], accZ = zero4(), accR[NTW], accr = zero4();
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    accS[k] = zero4();
    accR[k] = zero4();
  }
  const float* st0 = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
  if (!qrole) add_ST_tiles<D, M, NTW>(accS, st0, 0, 0, 1, sw, r16, g);
  if (zw) accZ = f32x4_t{1.f, 1.f, 1.f, 1.f} * st0[D * M + 16 * db + r16];
  auto stage_state = [&]() {
    if (qrole) return;
    float v4[4];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int mb = (sw + 4 * k) / DB;
      acc_to4(accS[k], v4);
      sp.put4(16 * db + r16, 16 * mb + 4 * g, v4);
    }
    if (zw && g == 0) sZ[16 * db + r16] = accZ[0];
  };
  stage_state();
  float lstart = 0.f;  // running sum of logA from the segment start to before the chunk

  auto chunk = [&](int b, int c0) {
    const int nv = min(CH, t1 - c0);
    const float lam = wave_incl_sum(ell[b]);
    const float last = __shfl(lam, 63, 64);
    __syncthreads();
    bq[b].stage_phi(qt, nv, nullptr, fm);
    bk[b].stage_phi(kt, nv, nullptr, fm);
    bv[b].stage_values(vt);
    bd[b].stage_values(ot);
    if (w == 0) {
      slam[l] = lam;
      sF[l] = exp_nat(last - lam);
    }
    fetch(b, c0 + 2 * CH);
    __syncthreads();

    if (qrole) {
      const int il = 16 * w + r16;
      const bool row_ok = il < nv;
      const float lam_i = slam[il], e_i = exp_nat(lam_i);
      Frag<P::Q> qf[D / 32];
      Frag<P::DO> dof[M / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) qf[s] = qt.template frag<P::Q>(il, 32 * s, g);
#pragma unroll
      for (int s = 0; s < M / 32; ++s) dof[s] = ot.template frag<P::DO>(il, 32 * s, g);

      // intra-chunk tiles, [j][i] with j = 16jb + 4g + r
      f32x4_t wt[4], pt[4];
      float dpA = 0.f, dpP = 0.f;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4(), p = zero4(), e = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s) mmaf<P::K, P::Q>(a, kt.template frag<P::K>(16 * jb + r16, 32 * s, g), qf[s]);
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mmaf<P::V, P::DO>(p, vt.template frag<P::V>(16 * jb + r16, 32 * s, g), dof[s]);
          const float4 lj = *reinterpret_cast<const float4*>(&slam[16 * jb + 4 * g]);
          const float ljv[4] = {lj.x, lj.y, lj.z, lj.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool on = jb < w || 4 * g + r <= r16;
            e[r] = on ? exp_nat(lam_i - ljv[r]) : 0.f;
            dpA += a[r] * e[r];
            dpP += a[r] * e[r] * p[r];
          }
        }
        wt[jb] = e;
        pt[jb] = p;
      }
      dpA = sum_over_g(dpA);
      dpP = sum_over_g(dpP);

      // state terms: U = S dO_i ([d][i]), phi(Q_i).Z and phi(Q_i).U
      f32x4_t U[DB];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        f32x4_t u = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::S, P::DO>(u, sp.template frag<P::S>(16 * d0 + r16, 32 * s, g), dof[s]);
        U[d0] = u;
      }
      float qv[DB][4], zv[DB][4], pu = 0.f, pz = 0.f;
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        qt.get4(il, 16 * d0 + 4 * g, qv[d0]);
        const float4 z4 = *reinterpret_cast<const float4*>(&sZ[16 * d0 + 4 * g]);
        zv[d0][0] = z4.x; zv[d0][1] = z4.y; zv[d0][2] = z4.z; zv[d0][3] = z4.w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pu += qv[d0][r] * U[d0][r];
          pz += qv[d0][r] * zv[d0][r];
        }
      }
      pu = sum_over_g(pu);
      pz = sum_over_g(pz);
      const float den = dpA + e_i * pz;
      const float inv = row_ok ? 1.f / den : 0.f;
      const float odo = row_ok ? (dpP + e_i * pu) * inv : 0.f;  // O_i . dO_i

      // W[j][i] = exp(lam_i - lam_j) (dO_i.V_j - O_i.dO_i), then sum_j W phi(K_j)
      Frag<P::W> wf[2];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pt[jb][r] = wt[jb][r] * (pt[jb][r] - odo);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) wf[p] = acc2frag<P::W>(pt[2 * p], pt[2 * p + 1]);
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p <= w) mmaf<P::K, P::W>(acc, kt.template tfrag_acc<P::K>(32 * p, 16 * d0, g, r16), wf[p]);
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dpq = (acc[r] + e_i * (U[d0][r] - odo * zv[d0][r])) * inv;
          o[r] = dpq * dfeat(qv[d0][r], fm);
        }
        if (row_ok) IO<T>::store4(dQ + offD + (size_t)(c0 + il) * D + 16 * d0 + 4 * g, o);
      }
      const float cc = -odo * inv;
      if (g == 0 && row_ok) gc[(size_t)bh * N + c0 + il] = make_float2(inv, cc);
      // [g_i | c_i] weighted to the segment start
      const float sc = row_ok ? exp_nat(lstart + lam_i) : 0.f;
#pragma unroll
      for (int mm = 0; mm < M / 4; mm += 4) {
        float dv[4];
        ot.get4(il, g * (M / 4) + mm, dv);
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] *= inv * sc;
        gt.put4(il, g * (M / 4) + mm, dv);
      }
      if (g == 0) gt.put1(il, M, cc * sc);
    } else {
      // state after the chunk: S^T = exp(lam_last) S^T + V^T diag(f) phi(K), in registers
      const float dec = exp_nat(last);
#pragma unroll
      for (int k = 0; k < NTW; ++k) accS[k] *= dec;
      accZ *= dec;
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const Frag<P::K> kb = scale_frag<P::K>(kt.template tfrag<P::K>(32 * s, 16 * db, g, r16), &sF[32 * s + 8 * g]);
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          const int mb = (sw + 4 * k) / DB;
          mmaf<P::V, P::K>(accS[k], vt.template tfrag<P::V>(32 * s, 16 * mb, g, r16), kb);
        }
        if (zw) mmaf<1, P::K>(accZ, ones, kb);
      }
    }
    __syncthreads();  // [g | c] complete; the query rows are done with S, Z of this chunk

    if (!qrole) {
      stage_state();  // read again only after the next chunk's first barrier
      // reverse aggregate: R^T += [g|c]^T phi(Q) (weighted rows)
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const Frag<P::Q> qb = qt.template tfrag<P::Q>(32 * s, 16 * db, g, r16);
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          const int mb = (sw + 4 * k) / DB;
          mmaf<P::G, P::Q>(accR[k], gt.template tfrag<P::G>(32 * s, 16 * mb, g, r16), qb);
        }
        if (zw) mmaf<P::G, P::Q>(accr, gt.template tfrag<P::G>(32 * s, M, g, r16), qb);
      }
    }
    lstart += last;
  };
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(0, c0);
    if (c0 + CH < t1) chunk(1, c0 + CH);
  }
  if (!qrole) {
    float* out = ragg + ((size_t)bh * nseg + seg) * SV;
    store_ST_tiles<D, M, NTW>(out, accR, sw, r16, g);
    if (zw && g == 0) out[D * M + 16 * db + r16] = accr[0];
  }
  if (tid == 0) dlam[(size_t)bh * nseg + seg] = lstart;
}

// Incoming reverse states, in place: ragg[bh][s] <- R+_s, the reverse state
// arriving at the end of segment s, with R+_{nseg-1} = (dS_N, dZ_N) or zero
// and R+_{s-1} = ragg_s + exp(dlam_s) R+_s; R+_{-1} (the gradient of the
// initial state) goes to dS0/dZ0 when given.
template <int D, int M>
__global__ __launch_bounds__(NT) void k_dscan_rev(float* __restrict__ ragg, const float* __restrict__ dlam,
                                                   const float* __restrict__ dSN, const float* __restrict__ dZN,
                                                   float* __restrict__ dS0, float* __restrict__ dZ0, int nseg) {
  constexpr int SV = D * M + D, BT = 16;
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NT + threadIdx.x;
  if (e >= SV) return;
  float run = 0.f;
  if (e < D * M) {
    if (dSN) run = dSN[(size_t)bh * D * M + e];
  } else {
    if (dZN) run = dZN[(size_t)bh * D + (e - D * M)];
  }
  float* a = ragg + (size_t)bh * nseg * SV + e;
  const float* dl = dlam + (size_t)bh * nseg;
  for (int s1 = nseg; s1 > 0; s1 -= BT) {
    const int s0 = s1 - BT;
    float v[BT], f[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      v[j] = s0 + j >= 0 ? a[(size_t)(s0 + j) * SV] : 0.f;
      f[j] = s0 + j >= 0 ? exp_nat(dl[s0 + j]) : 1.f;
    }
#pragma unroll
    for (int j = BT - 1; j >= 0; --j) {
      if (s0 + j >= 0) {
        a[(size_t)(s0 + j) * SV] = run;
        run = v[j] + f[j] * run;
      }
    }
  }
  if (dS0) {
    if (e < D * M)
      dS0[(size_t)bh * D * M + e] = run;
    else
      dZ0[(size_t)bh * D + (e - D * M)] = run;
  }
}

// --------------------------------------------------------- backward: keys
// Key pass over one segment in reverse chunk order, from the incoming
// reverse state R+ of the segment (entry seg of the scanned `rin`).  Per
// chunk, for the wave's key rows j (f_j = exp(lam_last - lam_j)):
//   dV_j = sum_{i>=j} exp(lam_i - lam_j) (phi(Q_i).phi(K_j)) g_i + f_j R+^T phi(K_j),
//   dphiK_j = sum_{i>=j} exp(lam_i - lam_j) (g_i.V_j + c_i) phi(Q_i) + f_j (R+ V_j + r+),
// with g_i = dO_i / den_i and (1/den_i, c_i) from the query pass; then
// R+ <- exp(lam_last) R+ + sum_i exp(lam_i) phi(Q_i) [g_i | c_i]^T for the
// chunk before.  With x_j = -phi(K_j).dphiK_j, dla[j] gets the running sum
// of x over the segment's tokens from j on (plus, in the last segment, the
// final-state term <[dS_N|dZ_N], [S_N|Z_N]> with S_N checkpoint entry nseg),
// and xseg[bh][seg] the segment's total; k_dla_fix adds the later segments'.
// Eight wavefronts in two roles, one of each per SIMD: wavefront rb (0-3)
// forms dV of key rows 16rb.., wavefront 4 + rb dphiK of the same rows (the
// attention tiles for dV, the dO.V tiles for dK); the tiles of R+ are spread
// over all eight.
template <typename T, int D, int M>
__global__ __launch_bounds__(2 * NT) void k_dbkv(const T* __restrict__ Q, const T* __restrict__ K,
                                                  const T* __restrict__ V, const T* __restrict__ dO,
                                                  const float* __restrict__ logA, const float2* __restrict__ gc,
                                                  const float* __restrict__ rin, const float* __restrict__ ckpt,
                                                  const float* __restrict__ dSN, const float* __restrict__ dZN,
                                                  T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ dla,
                                                  float* __restrict__ xseg, int N, int L, int nseg, int fm) {
  using P = DPrec<T>;
  constexpr int NTH = 2 * NT, DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NRW = DB * MB < 8 ? DB * MB : 8;  // wavefronts holding tiles of R+
  constexpr int NTR = DB * MB / NRW;              // tiles per holder: t = w + NRW k
  static_assert(NRW % DB == 0, "a holder's tiles share one feature block");
  __shared__ Planes<P::Q, CH, D> qt;
  __shared__ Planes<P::K, CH, D> kt;
  __shared__ Planes<P::V, CH, M> vt;
  __shared__ Planes<P::DO, CH, M> ot;
  __shared__ Planes<P::G, CH, M + 16> gt;  // exp(lam_i) [g_i | c_i | 0]
  __shared__ Planes<P::R, D, M> rp;        // R+, [d][m]
  __shared__ alignas(16) float sr[D];      // r+
  __shared__ alignas(16) float slam[CH];
  __shared__ alignas(16) float sInv[CH];
  __shared__ alignas(16) float sC[CH];
  __shared__ alignas(16) float sX[CH];  // x_j of the chunk just processed

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const bool vrole = w < 4;  // dV wavefront, else dK
  const int rb = w & 3;      // key row block
  const int db = w % DB;     // feature block of the wave's R+ tiles
  const bool rhold = w < NRW, zw = w < DB;
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;
  const float* la = logA + (size_t)bh * N;
  const float2* gch = gc + (size_t)bh * N;
  gt.zero_cols(M + 1, M + 16, NTH);

  // running sum of x from the segment's end (wave 0); the last segment starts it at the final-state term
  float carry = 0.f;
  if (seg == nseg - 1 && dSN) {
    const float* sn = ckpt + ((size_t)bh * (nseg + 1) + nseg) * SV;
    float acc = 0.f;
    for (int e = tid; e < SV; e += NTH)
      acc += (e < D * M ? dSN[(size_t)bh * D * M + e] : dZN[(size_t)bh * D + e - D * M]) * sn[e];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (l == 0) sX[w] = acc;
    __syncthreads();
    carry = ((sX[0] + sX[1]) + (sX[2] + sX[3])) + ((sX[4] + sX[5]) + (sX[6] + sX[7]));
    __syncthreads();
  }
  int pend_c0 = -1, pend_nv = 0;  // chunk whose x values wait in sX
  auto flush_x = [&]() {          // wave 0: dla of the pending chunk = suffix sums of x + carry
    if (w != 0 || pend_c0 < 0) return;
    const float x = sX[l];
    const float sfx = __shfl(wave_incl_sum(__shfl(x, 63 - l, 64)), 63 - l, 64);  // sum over lanes >= l
    if (l < pend_nv) dla[(size_t)bh * N + pend_c0 + l] = sfx + carry;
    carry += __shfl(sfx, 0, 64);
  };

  const int nchunk = (t1 - t0 + CH - 1) / CH;
  // a tensor with fewer vectors per chunk than threads goes to one half of the workgroup
  constexpr int OD_ = RowBuf<T, CH, D, NTH>::VEC < NTH ? NTH / 2 : 0;
  constexpr int OM_ = RowBuf<T, CH, M, NTH>::VEC < NTH ? NTH / 2 : 0;
  RowBuf<T, CH, D, NTH> bq[2];
  RowBuf<T, CH, D, NTH, OD_> bk[2];
  RowBuf<T, CH, M, NTH> bv[2];
  RowBuf<T, CH, M, NTH, OM_> bd[2];
  float ell[2];
  float2 gcl[2];
  auto fetch = [&](int b, int ci) {
    if (ci < 0) return;
    const int c0 = t0 + ci * CH, nv = min(CH, t1 - c0);
    bq[b].load(Q + offD + (size_t)c0 * D, nv);
    bk[b].load(K + offD + (size_t)c0 * D, nv);
    bv[b].load(V + offM + (size_t)c0 * M, nv);
    bd[b].load(dO + offM + (size_t)c0 * M, nv);
    ell[b] = load_ell(la, c0, nv);
    gcl[b] = l < nv ? gch[c0 + l] : make_float2(0.f, 0.f);
  };
  fetch(0, nchunk - 1);
  fetch(1, nchunk - 2);

  // R+ tiles of this wave in the S^T layout: accR[k][r] = R[16db + r16][16mb + 4g + r], t = w + NRW k
  f32x4_t accR[NTR], accr = zero4();
  auto rmb = [&](int k) { return (w + NRW * k) / DB; };
  {
    const float* r0 = rin + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      accR[k] = zero4();
      if (rhold) {
        const float4 a = *reinterpret_cast<const float4*>(r0 + (16 * db + r16) * M + 16 * rmb(k) + 4 * g);
        accR[k] = f32x4_t{a.x, a.y, a.z, a.w};
      }
    }
    if (zw) accr = f32x4_t{1.f, 1.f, 1.f, 1.f} * r0[D * M + 16 * db + r16];
  }
  auto stage_R = [&]() {
    if (rhold) {
      float v4[4];
#pragma unroll
      for (int k = 0; k < NTR; ++k) {
        acc_to4(accR[k], v4);
        rp.put4(16 * db + r16, 16 * rmb(k) + 4 * g, v4);
      }
    }
    if (zw && g == 0) sr[16 * db + r16] = accr[0];
  };

  auto chunk = [&](int b, int ci) {
    const int c0 = t0 + ci * CH, nv = min(CH, t1 - c0);
    const float lam = wave_incl_sum(ell[b]);
    const float last = __shfl(lam, 63, 64);
    const float2 gcv = gcl[b];
    __syncthreads();
    flush_x();
    stage_R();
    bq[b].stage_phi(qt, nv, nullptr, fm);
    bk[b].stage_phi(kt, nv, nullptr, fm);
    bv[b].stage_values(vt);
    // dO, and [g | c] weighted by exp(lam_i), from the same registers
    {
      auto& bdo = bd[b];
      if (bdo.owns()) {
#pragma unroll
        for (int n = 0; n < bdo.CNT; ++n) {
          const int row = bdo.row_of(n), col = bdo.col_of(n);
          float x[IO<T>::E];
          IO<T>::unpack(bdo.r[n], x);
          ot.template put<IO<T>::E>(row, col, x);
          const float lr = __shfl(lam, row, 64), ir = __shfl(gcv.x, row, 64), cr = __shfl(gcv.y, row, 64);
          const float sc = exp_nat(lr) * ir;
#pragma unroll
          for (int e = 0; e < IO<T>::E; ++e) x[e] *= sc;
          gt.template put<IO<T>::E>(row, col, x);
          if (col == 0) gt.put1(row, M, cr * exp_nat(lr));
        }
      }
    }
    if (w == 0) {
      slam[l] = lam;
      sInv[l] = gcv.x;
      sC[l] = gcv.y;
    }
    fetch(b, ci - 2);
    __syncthreads();

    const int jl = 16 * rb + r16;
    const bool row_ok = jl < nv;
    const float lam_j = slam[jl], f_j = exp_nat(last - lam_j);
    // tiles [i][j] with i = 16ib + 4g + r >= j: the attention A (dV role) or dO.V (dK role), weighted
    f32x4_t tw[4];
    {
      Frag<P::K> kf[D / 32];
      Frag<P::V> vf[M / 32];
      if (vrole) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) kf[s] = kt.template frag<P::K>(jl, 32 * s, g);
      } else {
#pragma unroll
        for (int s = 0; s < M / 32; ++s) vf[s] = vt.template frag<P::V>(jl, 32 * s, g);
      }
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4_t a = zero4();
        if (ib >= rb) {
          if (vrole) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s) mmaf<P::Av, P::Av>(a, qt.template frag<P::Av>(16 * ib + r16, 32 * s, g), kf[s]);
          } else {
#pragma unroll
            for (int s = 0; s < M / 32; ++s)
              mmaf<P::DO, P::V>(a, ot.template frag<P::DO>(16 * ib + r16, 32 * s, g), vf[s]);
          }
          const float4 li = *reinterpret_cast<const float4*>(&slam[16 * ib + 4 * g]);
          const float4 iv = *reinterpret_cast<const float4*>(&sInv[16 * ib + 4 * g]);
          const float4 cv = *reinterpret_cast<const float4*>(&sC[16 * ib + 4 * g]);
          const float liv[4] = {li.x, li.y, li.z, li.w}, ivv[4] = {iv.x, iv.y, iv.z, iv.w},
                      cvv[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool on = ib > rb || 4 * g + r >= r16;
            const float e = on ? exp_nat(liv[r] - lam_j) : 0.f;
            a[r] = vrole ? a[r] * e * ivv[r] : e * (a[r] * ivv[r] + cvv[r]);
          }
        }
        tw[ib] = a;
      }
      Frag<P::W> wf[2];
      if (vrole) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const Frag<P::Wv> f = acc2frag<P::Wv>(tw[2 * p], tw[2 * p + 1]);
#pragma unroll
          for (int q = 0; q < P::Wv; ++q) wf[p].p[q] = f.p[q];
        }
      } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) wf[p] = acc2frag<P::W>(tw[2 * p], tw[2 * p + 1]);
      }
      if (vrole) {
        // dV_j[m] = sum_i dO_i[m] aw[i][j] + f_j (R+^T phi(K_j))[m]
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4_t st = zero4(), acc = zero4();
#pragma unroll
          for (int s = 0; s < D / 32; ++s) mmaf<P::R, P::Kv>(st, rp.template tfrag<P::R>(32 * s, 16 * mb, g, r16), kf[s]);
#pragma unroll
          for (int p = 0; p < 2; ++p)
            if (2 * p + 1 >= rb) mmaf<P::DO, P::Wv>(acc, ot.template tfrag_acc<P::DO>(32 * p, 16 * mb, g, r16), wf[p]);
          if (row_ok) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = acc[r] + f_j * st[r];
            IO<T>::store4(dV + offM + (size_t)(c0 + jl) * M + 16 * mb + 4 * g, o);
          }
        }
      } else {
        // dphiK_j[d] = sum_i phi(Q_i)[d] ww[i][j] + f_j ((R+ V_j)[d] + r+[d])
        float xk = 0.f;
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
          f32x4_t st = zero4(), acc = zero4();
#pragma unroll
          for (int s = 0; s < M / 32; ++s) mmaf<P::R, P::V>(st, rp.template frag<P::R>(16 * d0 + r16, 32 * s, g), vf[s]);
#pragma unroll
          for (int p = 0; p < 2; ++p)
            if (2 * p + 1 >= rb) mmaf<P::Q, P::W>(acc, qt.template tfrag_acc<P::Q>(32 * p, 16 * d0, g, r16), wf[p]);
          float kv[4];
          kt.get4(jl, 16 * d0 + 4 * g, kv);
          const float4 r4 = *reinterpret_cast<const float4*>(&sr[16 * d0 + 4 * g]);
          const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dpk = acc[r] + f_j * (st[r] + rr[r]);
            xk += kv[r] * dpk;
            o[r] = dpk * dfeat(kv[r], fm);
          }
          if (row_ok) IO<T>::store4(dK + offD + (size_t)(c0 + jl) * D + 16 * d0 + 4 * g, o);
        }
        xk = sum_over_g(xk);
        if (g == 0) sX[jl] = row_ok ? -xk : 0.f;
      }
    }
    pend_c0 = c0;
    pend_nv = nv;

    // R+ for the chunk before
    const float dec = exp_nat(last);
#pragma unroll
    for (int k = 0; k < NTR; ++k) accR[k] *= dec;
    accr *= dec;
    if (rhold) {
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const Frag<P::Q> qb = qt.template tfrag<P::Q>(32 * s, 16 * db, g, r16);
#pragma unroll
        for (int k = 0; k < NTR; ++k) mmaf<P::G, P::Q>(accR[k], gt.template tfrag<P::G>(32 * s, 16 * rmb(k), g, r16), qb);
        if (zw) mmaf<P::G, P::Q>(accr, gt.template tfrag<P::G>(32 * s, M, g, r16), qb);
      }
    }
  };
  for (int ci = nchunk - 1; ci >= 0; ci -= 2) {
    chunk(0, ci);
    if (ci - 1 >= 0) chunk(1, ci - 1);
  }
  __syncthreads();
  flush_x();
  if (tid == 0) xseg[(size_t)bh * nseg + seg] = carry;
}

// dla over segment seg += the totals xseg of the later segments (summed in
// segment order).
__global__ __launch_bounds__(NT) void k_dla_fix(float* __restrict__ dla, const float* __restrict__ xseg, int N,
                                                 int L, int nseg) {
  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  if (seg == nseg - 1) return;
  float off = 0.f;
  for (int s = seg + 1; s < nseg; ++s) off += xseg[(size_t)bh * nseg + s];
  const int t0 = seg * L, t1 = min(N, t0 + L);
  float* x = dla + (size_t)bh * N;
  for (int t = t0 + (int)threadIdx.x; t < t1; t += NT) x[t] += off;
}

}  // namespace la
