// la_bwd2.h -- the causal backward in two passes over the checkpoint's
// segments ("Transformers are RNNs -- part 2/3", section 3.3.1, eq. 13-15,
// with the denominator's share by the quotient rule).
//
// With g_i = dO_i / den_i and c_i = -(O_i . dO_i) / den_i the gradients are
//   dphi(Q_i) = S_i g_i + c_i Z_i                        (eq. 13, forward sum)
//   dphi(K_j) = sum_{i>=j} phi(Q_i) (g_i . V_j + c_i)    (eq. 14, backward sum)
//   dV_j      = sum_{i>=j} g_i (phi(Q_i) . phi(K_j))     (eq. 15, backward sum)
// i.e. eq. 13-15 on [V, 1] with upstream [g, c].  The backward sums run over
// the reverse state R = sum_{i>=j} phi(Q_i) g_i^T, r = sum_{i>=j} c_i phi(Q_i).
//
// Pass A (k_bq) walks each segment forward from its checkpoint state, as
// the forward did: it forms S_i, Z_i exactly (the state before the chunk plus
// the causal part of the chunk), recomputes den_i = phi(Q_i) . Z_i and
// O_i . dO_i = phi(Q_i)^T S_i dO_i / den_i in float32 -- so neither the stored
// O nor den is read, and g_i . V_j + c_i = (dO_i . V_j - O_i . dO_i) / den_i
// cancels exactly where V_j = O_i even for bf16 storage -- writes dQ and the
// per-token pair (1/den_i, O_i . dO_i), and sums the segment's exact reverse
// aggregate (R, r over its tokens).  The suffix sums of those aggregates
// (the final-state gradient dS_N, dZ_N added) give every segment the
// reverse state after its last token.  Pass B (k_bkv) walks each segment
// backwards from that state and forms dK, dV from the stored pairs.
//
// Each pass carries one state, so a workgroup needs one state in registers
// and LDS.  Chunks of 32 tokens, four wavefronts in two roles:
//   pass A  waves 0, 1: query rows 16w..16w+15 (S_i dO_i, Z_i, den_i,
//                       O_i . dO_i, dQ, the row [g_i | c_i]);
//           waves 2, 3: the chunk's state update S += phi(K)^T V, Z +=
//                       phi(K)^T 1 in registers, and the previous chunk's
//                       share of the reverse aggregate [g | c]^T phi(Q).
//   pass B  waves 0, 1: key rows 16w..16w+15 (dK, dV);
//           waves 2, 3: the chunk's share of the reverse state, R^T +=
//                       [g | c]^T phi(Q), in registers.
// Two barriers per chunk: after staging, and after phase 1; the state the
// next chunk reads is staged, and the next chunk's operands, after it.
#pragma once

#include "la_kernels.h"

namespace la {

constexpr int CB2 = 32;  // chunk of the two-pass backward

// ===================================================================== B-A
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_bq(const T* __restrict__ Q, const T* __restrict__ K,
                                            const T* __restrict__ V, const T* __restrict__ dO,
                                            const float* __restrict__ ckpt, T* __restrict__ dQ,
                                            float2* __restrict__ gc, float* __restrict__ ragg, int N, int L, int nseg,
                                            int fm) {
  using P = Prec<T>;
  constexpr int CB = CB2;
  constexpr int DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NTS = DB * MB / 2;        // S^T tiles per update wave
  constexpr int NZS = DB / 2;             // Z blocks per update wave
  constexpr int NTR = (MB + 1) * DB / 2;  // [R | r]^T tiles per update wave
  __shared__ Planes<P::NK, CB, D> kt;           // phi(K)
  __shared__ Planes<P::NV, CB, M> vt;           // V
  __shared__ Planes<P::NDO, CB, M> ot;          // dO
  __shared__ Planes<P::NQ, CB, D> qt[2];        // phi(Q) of this chunk and the previous one
  __shared__ Planes<P::NG, CB, M + 16> gt[2];   // [g | c | 0] of this chunk and the previous one
  __shared__ Planes<P::NS, D, M> sp;            // S before this chunk, [d][m]
  __shared__ alignas(16) float sZ[D];           // Z before this chunk

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const bool qrole = w < 2;
  const int so = w - 2;  // rank among the update waves
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;
  const Frag<1> ones = ones_frag();
  gt[0].zero_cols(M + 1, M + 16);
  gt[1].zero_cols(M + 1, M + 16);

  // update-wave tiles: S^T tile k: t = so + 2k, feature block t % DB, value block t / DB;
  // [R | r]^T tile k: t = so + 2k, feature block t % DB, value block t / DB (block MB holds r)
  auto tdb = [&](int k) { return (so + 2 * k) % DB; };
  auto tmb = [&](int k) { return (so + 2 * k) / DB; };

  const int nchunk = (t1 - t0 + CB - 1) / CB;
  constexpr int OQ_ = RowBuf<T, CB, D>::VEC < NT ? NT / 2 : 0;
  constexpr int OM_ = RowBuf<T, CB, M>::VEC < NT ? NT / 2 : 0;
  RowBuf<T, CB, D> bq;
  RowBuf<T, CB, D, NT, OQ_> bk;
  RowBuf<T, CB, M> bv;
  RowBuf<T, CB, M, NT, OM_> bd;
  auto fetch = [&](int c0) {
    const int nv = min(CB, t1 - c0);
    bq.load(Q + offD + (size_t)c0 * D, nv);
    bk.load(K + offD + (size_t)c0 * D, nv);
    bv.load(V + offM + (size_t)c0 * M, nv);
    bd.load(dO + offM + (size_t)c0 * M, nv);
  };
  fetch(t0);

  f32x4_t accS[NTS], accR[NTR];
  float zz[NZS];
#pragma unroll
  for (int k = 0; k < NTR; ++k) accR[k] = zero4();
  auto stage_S = [&]() {
    float v4[4];
#pragma unroll
    for (int k = 0; k < NTS; ++k) {
      acc_to4(accS[k], v4);
      sp.put4(16 * tdb(k) + r16, 16 * tmb(k) + 4 * g, v4);
    }
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < NZS; ++j) sZ[16 * (so + 2 * j) + r16] = zz[j];
    }
  };
  if (!qrole) {  // the state before the segment: the forward's checkpoint entry
    const float* st = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTS; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(st + (16 * tdb(k) + r16) * M + 16 * tmb(k) + 4 * g);
      accS[k] = f32x4_t{a.x, a.y, a.z, a.w};
    }
#pragma unroll
    for (int j = 0; j < NZS; ++j) zz[j] = st[D * M + 16 * (so + 2 * j) + r16];
    stage_S();
  }

  // [R | r]^T += [g | c]^T phi(Q) over the chunk staged in buffer b
  auto rproduct = [&](int b) {
#pragma unroll
    for (int k = 0; k < NTR; ++k)
      mmaf<P::dR, P::dR>(accR[k], gt[b].template tfrag<P::dR>(0, 16 * tmb(k), g, r16),
                         qt[b].template tfrag<P::dR>(0, 16 * tdb(k), g, r16));
  };

  for (int ci = 0; ci < nchunk; ++ci) {
    const int c0 = t0 + ci * CB, cur = ci & 1;
    const int nv = min(CB, t1 - c0);
    // ---- stage this chunk (the barrier ending the previous phase 1 separates the previous reads)
    bq.template stage_phi<P::NQ, CB, D, 8, 0>(qt[cur], nv, nullptr, fm);
    bk.template stage_phi<P::NK, CB, D, 8, 0>(kt, nv, nullptr, fm);
    bv.stage_values(vt);
    bd.stage_values(ot);
    if (ci + 1 < nchunk) fetch(c0 + CB);
    __syncthreads();

    if (qrole) {
      // ================ query rows il: S_i = S + sum_{j<=i} phi(K_j) V_j^T, Z_i likewise
      const int ib = w, il = 16 * ib + r16;
      const bool row_ok = il < nv;
      constexpr int NO = cmax(P::Bt, P::U1_b);
      Frag<NO> dof[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) dof[s] = ot.template frag<NO>(il, 32 * s, g);
      // (V_j . dO_i) for j <= i as a B operand under the accumulator map, and the mask [j <= i]
      Frag<P::U2> btf;
      Frag<1> onef;
      {
        f32x4_t bt[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          f32x4_t a = zero4();
          if (jb <= ib) {
#pragma unroll
            for (int s = 0; s < M / 32; ++s)
              mmaf<P::Bt, P::Bt>(a, vt.template frag<P::Bt>(16 * jb + r16, 32 * s, g), dof[s]);
            if (jb == ib) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > r16) a[r] = 0.f;  // j > i
            }
          }
          bt[jb] = a;
        }
        btf = acc2frag<P::U2>(bt[0], bt[1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
          onef.p[0][e] = j <= il ? (__bf16)1.0f : (__bf16)0.0f;
        }
      }
      f32x4_t U[DB], ZC[DB];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        f32x4_t u = zero4(), zc = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::U1_a, P::U1_b>(u, sp.template frag<P::U1_a>(16 * d0 + r16, 32 * s, g), dof[s]);
        constexpr int NKA = cmax(P::U2, P::Zc);
        const Frag<NKA> kfa = kt.template tfrag_acc<NKA>(0, 16 * d0, g, r16);
        mmaf<P::U2, P::U2>(u, kfa, btf);
        mmaf<P::Zc, 1>(zc, kfa, onef);
        const float4 z4 = *reinterpret_cast<const float4*>(&sZ[16 * d0 + 4 * g]);
        zc += f32x4_t{z4.x, z4.y, z4.z, z4.w};
        U[d0] = u;    // S_i dO_i   [d][i]
        ZC[d0] = zc;  // Z_i        [d][i]
      }
      float pu = 0.f, pz = 0.f;
      float qv[DB][4];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        qt[cur].get4(il, 16 * d0 + 4 * g, qv[d0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pu += qv[d0][r] * U[d0][r];
          pz += qv[d0][r] * ZC[d0][r];
        }
      }
      pu = sum_over_g(pu);  // phi(Q_i)^T S_i dO_i = num_i . dO_i
      pz = sum_over_g(pz);  // phi(Q_i) . Z_i = den_i
      const float invz = row_ok ? 1.f / pz : 0.f;
      const float odo = row_ok ? pu * invz : 0.f;  // O_i . dO_i
      if (row_ok) {
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (U[d0][r] - ZC[d0][r] * odo) * invz * dfeat(qv[d0][r], fm);
          IO<T>::store4(dQ + offD + (size_t)(c0 + il) * D + 16 * d0 + 4 * g, o);
        }
        if (g == 0) gc[(size_t)bh * N + c0 + il] = make_float2(invz, odo);
      }
      // row i of [g | c]: g_i = dO_i / den_i over this lane's quarter of the features, c_i = -(O_i . dO_i) / den_i
#pragma unroll
      for (int mm = 0; mm < M / 4; mm += 4) {
        float dv[4];
        ot.get4(il, g * (M / 4) + mm, dv);
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] *= invz;
        gt[cur].put4(il, g * (M / 4) + mm, dv);
      }
      if (g == 0) gt[cur].put1(il, M, -odo * invz);
    } else {
      // ================ the previous chunk's reverse aggregate, then the state update
      if (ci > 0) rproduct(cur ^ 1);
      constexpr int NKB = cmax(P::dS_b, P::Zc);
#pragma unroll
      for (int k = 0; k < NTS; ++k)
        mmaf<P::dS_a, P::dS_b>(accS[k], vt.template tfrag<P::dS_a>(0, 16 * tmb(k), g, r16),
                               kt.template tfrag<NKB>(0, 16 * tdb(k), g, r16));
#pragma unroll
      for (int j = 0; j < NZS; ++j) {
        f32x4_t dz = zero4();
        mmaf<1, P::Zc>(dz, ones, kt.template tfrag<NKB>(0, 16 * (so + 2 * j), g, r16));
        zz[j] += dz[0];
      }
    }
    __syncthreads();
    if (!qrole) stage_S();  // S, Z before the next chunk
  }
  if (!qrole && nchunk > 0) rproduct((nchunk - 1) & 1);
  // the segment's reverse aggregate (sum over its tokens of phi(Q_i) g_i^T, c_i phi(Q_i)), [d][m] then r,
  // for the segments before it; segment 0's is not needed
  if (!qrole && seg > 0) {
    float* out = ragg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int db = tdb(k), mb = tmb(k);
      if (mb < MB) {
        *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
            make_float4(accR[k][0], accR[k][1], accR[k][2], accR[k][3]);
      } else if (g == 0) {
        out[D * M + 16 * db + r16] = accR[k][0];  // row M of the tile: r
      }
    }
  }
}

// ===================================================================== B-B
// Reverse walk of a segment: key rows form dK, dV from the reverse state
// after the chunk (R, r: the final-state gradient plus the later segments'
// aggregates plus the later chunks of this segment) and the chunk's own
// causal part; the update waves carry R, r to before the chunk.  The
// sequence's first segment writes the reverse state carried through token 1:
// the gradient of the initial state (dS0, dZ0).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_bkv(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, const T* __restrict__ dO,
                                             const float2* __restrict__ gc, const float* __restrict__ ragg,
                                             const float* __restrict__ dSN, const float* __restrict__ dZN,
                                             T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ dS0,
                                             float* __restrict__ dZ0, int N, int L, int nseg, int scanned, int fm) {
  using P = Prec<T>;
  constexpr int CB = CB2;
  constexpr int DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NTR = DB * MB / 2;  // R^T tiles per update wave
  constexpr int NZR = DB / 2;       // r blocks per update wave
  __shared__ Planes<P::NQ, CB, D> qt;          // phi(Q)
  __shared__ Planes<P::NK, CB, D> kt;          // phi(K)
  __shared__ Planes<P::NV, CB, M> vt;          // V
  __shared__ Planes<P::NDO, CB, M> ot;         // dO
  __shared__ Planes<P::NG, CB, M + 16> gt;     // [g | c | 0]
  __shared__ Planes<P::NR, D, M> rp;           // R after this chunk, [d][m]
  __shared__ alignas(16) float sr[D];          // r after this chunk
  __shared__ alignas(16) float sInv[CB];       // 1 / den_i (0 past the end)
  __shared__ alignas(16) float sOdo[CB];       // O_i . dO_i (0 past the end)

  const int seg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const bool krole = w < 2;
  const int so = w - 2;
  const size_t offD = (size_t)bh * N * D, offM = (size_t)bh * N * M;
  gt.zero_cols(M + 1, M + 16);
  auto tdb = [&](int k) { return (so + 2 * k) % DB; };
  auto tmb = [&](int k) { return (so + 2 * k) / DB; };

  const int nchunk = (t1 - t0 + CB - 1) / CB;
  constexpr int OQ_ = RowBuf<T, CB, D>::VEC < NT ? NT / 2 : 0;
  constexpr int OM_ = RowBuf<T, CB, M>::VEC < NT ? NT / 2 : 0;
  RowBuf<T, CB, D> bq;
  RowBuf<T, CB, D, NT, OQ_> bk;
  RowBuf<T, CB, M> bv;
  RowBuf<T, CB, M, NT, OM_> bd;
  using BD = RowBuf<T, CB, M, NT, OM_>;
  float2 pgc = make_float2(0.f, 0.f);  // (1/den, O.dO) of token tid of the chunk (threads < CB)
  float pinv[BD::CNT];                  // 1/den of the rows of this thread's dO vectors
  auto fetch = [&](int c0) {
    const int nv = min(CB, t1 - c0);
    bq.load(Q + offD + (size_t)c0 * D, nv);
    bk.load(K + offD + (size_t)c0 * D, nv);
    bv.load(V + offM + (size_t)c0 * M, nv);
    bd.load(dO + offM + (size_t)c0 * M, nv);
    if (tid < CB) pgc = tid < nv ? gc[(size_t)bh * N + c0 + tid] : make_float2(0.f, 0.f);
    if (BD::owns()) {
#pragma unroll
      for (int i = 0; i < BD::CNT; ++i) {
        const int row = BD::row_of(i);
        pinv[i] = row < nv ? gc[(size_t)bh * N + c0 + row].x : 0.f;
      }
    }
  };
  fetch(t0 + (nchunk - 1) * CB);

  // reverse state after the segment: the final-state gradient plus the later segments' aggregates (entry seg
  // of the suffix sums when scanned, else their sum in segment order), summed through R's planes as scratch
  f32x4_t accR[NTR];
  float zr[NZR];
#pragma unroll
  for (int k = 0; k < NTR; ++k) accR[k] = zero4();
#pragma unroll
  for (int j = 0; j < NZR; ++j) zr[j] = 0.f;
  const float* rg = nseg > 1 ? ragg + (size_t)bh * nseg * SV : nullptr;
  const bool later = rg && seg + 1 < nseg;
  if (later || dSN) {
    // (scanned: entry s holds the sum over p > s)
    const int r0 = !later ? 0 : scanned ? seg : seg + 1, r1 = !later ? 0 : scanned ? seg + 1 : nseg;
    static_assert(sizeof(rp.v) >= SV * sizeof(float), "R planes too small to hold a float32 state");
    float* sbuf = reinterpret_cast<float*>(&rp.v[0][0][0]);
    sum_states<D, M, NT>(sbuf, dSN ? dSN + (size_t)bh * D * M : nullptr, dZN ? dZN + (size_t)bh * D : nullptr,
                         later ? rg : nullptr, r0, r1);
    __syncthreads();
    if (!krole) {
#pragma unroll
      for (int k = 0; k < NTR; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(sbuf + (16 * tdb(k) + r16) * M + 16 * tmb(k) + 4 * g);
        accR[k] = f32x4_t{a.x, a.y, a.z, a.w};
      }
#pragma unroll
      for (int j = 0; j < NZR; ++j) zr[j] = sbuf[D * M + 16 * (so + 2 * j) + r16];
    }
    __syncthreads();
  }
  auto stage_R = [&]() {
    float v4[4];
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      acc_to4(accR[k], v4);
      rp.put4(16 * tdb(k) + r16, 16 * tmb(k) + 4 * g, v4);
    }
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < NZR; ++j) sr[16 * (so + 2 * j) + r16] = zr[j];
    }
  };
  if (!krole) stage_R();

  for (int ci = nchunk - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * CB;
    const int nv = min(CB, t1 - c0);
    // ---- stage this chunk
    bq.template stage_phi<P::NQ, CB, D, 8, 0>(qt, nv, nullptr, fm);
    bk.template stage_phi<P::NK, CB, D, 8, 0>(kt, nv, nullptr, fm);
    bv.stage_values(vt);
    bd.stage_values(ot);
    // rows of [g | c]: g_i = dO_i / den_i from this thread's dO vectors, c_i = -(O_i . dO_i) / den_i
    if (BD::owns()) {
#pragma unroll
      for (int i = 0; i < BD::CNT; ++i) {
        float x[BD::E];
        IO<T>::unpack(bd.r[i], x);
#pragma unroll
        for (int e = 0; e < BD::E; ++e) x[e] *= pinv[i];
        gt.template put<BD::E>(BD::row_of(i), BD::col_of(i), x);
      }
    }
    if (tid < CB) {
      sInv[tid] = pgc.x;
      sOdo[tid] = pgc.y;
      gt.put1(tid, M, -pgc.y * pgc.x);
    }
    if (ci > 0) fetch(c0 - CB);
    __syncthreads();

    if (krole) {
      constexpr int NKT = cmax(P::At, P::VR);
      constexpr int NVT = cmax(P::Wt, P::KR_b);
      const int jb = w, jl = 16 * jb + r16;
      const bool row_ok = jl < nv;
      Frag<NKT> kfr[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kfr[s] = kt.template frag<NKT>(jl, 32 * s, g);
      Frag<NVT> vfr[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) vfr[s] = vt.template frag<NVT>(jl, 32 * s, g);
      // A_ij = phi(Q_i) . phi(K_j) and W_ij = (dO_i . V_j - O_i . dO_i) / den_i for i >= j (rows i, columns j)
      f32x4_t at[2], wt[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        f32x4_t a = zero4(), b = zero4();
        if (ib >= jb) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s)
            mmaf<P::At, P::At>(a, qt.template frag<P::At>(16 * ib + r16, 32 * s, g), kfr[s]);
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mmaf<P::Wt, P::Wt>(b, ot.template frag<P::Wt>(16 * ib + r16, 32 * s, g), vfr[s]);
          const float4 iv = *reinterpret_cast<const float4*>(&sInv[16 * ib + 4 * g]);
          const float4 od = *reinterpret_cast<const float4*>(&sOdo[16 * ib + 4 * g]);
          const float ivr[4] = {iv.x, iv.y, iv.z, iv.w}, odr[4] = {od.x, od.y, od.z, od.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            b[r] = (b[r] - odr[r]) * ivr[r];
            if (ib == jb && 4 * g + r < r16) {  // i < j
              a[r] = 0.f;
              b[r] = 0.f;
            }
          }
        }
        at[ib] = a;
        wt[ib] = b;
      }
      const Frag<P::dK> wfr = acc2frag<P::dK>(wt[0], wt[1]);
      const Frag<P::dV> afr = acc2frag<P::dV>(at[0], at[1]);
      // dK_j = (R V_j + r + sum_{i>=j} phi(Q_i) W_ij) phi'(K_j)
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        f32x4_t a = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::KR_a, P::KR_b>(a, rp.template frag<P::KR_a>(16 * d0 + r16, 32 * s, g), vfr[s]);
        mmaf<P::dK, P::dK>(a, qt.template tfrag_acc<P::dK>(0, 16 * d0, g, r16), wfr);
        if (row_ok) {
          float o[4], kv[4];
          kt.get4(jl, 16 * d0 + 4 * g, kv);
          const float4 r4 = *reinterpret_cast<const float4*>(&sr[16 * d0 + 4 * g]);
          const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (a[r] + rr[r]) * dfeat(kv[r], fm);
          IO<T>::store4(dK + offD + (size_t)(c0 + jl) * D + 16 * d0 + 4 * g, o);
        }
      }
      // dV_j = R^T phi(K_j) + sum_{i>=j} g_i A_ij
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t a = zero4();
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
          mmaf<P::VR, P::VR>(a, rp.template tfrag<P::VR>(32 * s, 16 * mb, g, r16), kfr[s]);
        mmaf<P::dV, P::dV>(a, gt.template tfrag_acc<P::dV>(0, 16 * mb, g, r16), afr);
        if (row_ok) {
          float o[4] = {a[0], a[1], a[2], a[3]};
          IO<T>::store4(dV + offM + (size_t)(c0 + jl) * M + 16 * mb + 4 * g, o);
        }
      }
    } else {
      // R^T += g^T phi(Q), r += phi(Q)^T c (row M of [g | c]) for the earlier chunks
#pragma unroll
      for (int k = 0; k < NTR; ++k)
        mmaf<P::dR, P::dR>(accR[k], gt.template tfrag<P::dR>(0, 16 * tmb(k), g, r16),
                           qt.template tfrag<P::dR>(0, 16 * tdb(k), g, r16));
#pragma unroll
      for (int j = 0; j < NZR; ++j) {
        f32x4_t dr = zero4();
        mmaf<P::dR, P::dR>(dr, gt.template tfrag<P::dR>(0, M, g, r16),
                           qt.template tfrag<P::dR>(0, 16 * (so + 2 * j), g, r16));
        zr[j] += dr[0];  // row M of the tile, on lanes g = 0
      }
    }
    __syncthreads();  // every wavefront is done with this chunk's LDS, and the key rows with R, r
    if (!krole) stage_R();
  }
  // the reverse state carried through the sequence's first token is the gradient of the initial state
  if (t0 == 0 && dS0 && !krole) {
#pragma unroll
    for (int k = 0; k < NTR; ++k)
      *reinterpret_cast<float4*>(dS0 + (size_t)bh * D * M + (16 * tdb(k) + r16) * M + 16 * tmb(k) + 4 * g) =
          make_float4(accR[k][0], accR[k][1], accR[k][2], accR[k][3]);
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < NZR; ++j) dZ0[(size_t)bh * D + 16 * (so + 2 * j) + r16] = zr[j];
    }
  }
}

}  // namespace la
