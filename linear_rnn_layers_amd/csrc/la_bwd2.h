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
// Writing q'_i = phi(Q_i) / den_i, every term that carries 1/den_i takes it
// from q': R = sum_i q'_i dO_i^T, r = -sum_i (O_i . dO_i) q'_i,
// phi(Q_i) (g_i . V_j + c_i) = q'_i (dO_i . V_j - O_i . dO_i) and
// g_i (phi(Q_i) . phi(K_j)) = dO_i (q'_i . phi(K_j)), so dO (exact in one bf16
// plane for bf16 storage) is the other operand and no g is staged.
//
// Pass A (k_bq) walks each segment forward from its checkpoint state, as
// the forward did: it forms S_i, Z_i exactly (the state before the chunk plus
// the causal part of the chunk), recomputes den_i = phi(Q_i) . Z_i and
// O_i . dO_i = phi(Q_i)^T S_i dO_i / den_i in float32 -- so neither the stored
// O nor den is read, and dO_i . V_j - O_i . dO_i cancels exactly where V_j = O_i
// even for bf16 storage -- writes dQ and the per-token pair (1/den_i,
// O_i . dO_i), and sums the segment's exact reverse aggregate (R, r over its
// tokens).  The suffix sums of those aggregates (the final-state gradient
// dS_N, dZ_N added) give every segment the reverse state after its last
// token.  Pass B (k_bkv) walks each segment backwards from that state and
// forms dK, dV from the stored pairs.
//
// Chunks of 64 tokens, four wavefronts in one role: wave w owns rows
// 16w..16w+15 of the chunk (query rows in pass A, key rows in pass B) and a
// quarter of the state's tiles (S^T and [R | r]^T in pass A, [R | r]^T in
// pass B).  Each pass carries one state in registers and stages it in LDS
// once per chunk.  Barriers per chunk: pass A three (after staging; after the
// query rows, whose q' and O.dO the aggregate product reads; after that
// product and the state update), pass B two (after staging; after the key
// rows and the reverse-state update, which read only this chunk's operands).
#pragma once

#include "la_kernels.h"

namespace la {

// -O.dO of row i as the extra columns M (and M + 1) of the dO planes, so that
// r is one more row block of [R | r]^T: for a one-plane dO (bf16 storage) the
// value is written as a rounded part in column M and its rounded residual in
// column M + 1 (their sum is float32-accurate), otherwise split into the
// planes of column M.
template <int NP, int ROWS, int COLS, int PAD>
__device__ __forceinline__ void put_neg_odo(Planes<NP, ROWS, COLS, PAD>& p, int row, int M, float odo) {
  const float x = -odo;
  if constexpr (NP == 1) {
    const __bf16 h = (__bf16)x;
    const __bf16 l = (__bf16)(x - (float)h);
    p.v[0][row][M] = __builtin_bit_cast(bf16_t, h);
    p.v[0][row][M + 1] = __builtin_bit_cast(bf16_t, l);
  } else {
    p.put1(row, M, x);
#pragma unroll
    for (int q = 0; q < NP; ++q) p.v[q][row][M + 1] = 0;
  }
}

// [R | r]^T += [dO | -O.dO]^T q' over one 64-token chunk: tiles t = w + 4k
// (t < the tile count) of the (M/16 + 1) x (D/16) tile grid, value block
// t / DB (block M/16 holds the r rows M, M + 1), feature block t % DB.  DB
// divides 4, so every tile of a wave has feature block w % DB and the q'
// fragment is read once per step for all of them.
template <typename T, int D, int M, int NTR, int NPO, int NPQ>
__device__ __forceinline__ void rproduct64(f32x4_t* accR, const Planes<NPO, CH, M + 16>& ot,
                                           const Planes<NPQ, CH, D>& qt, int w, int g, int r16) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NRT = (M / 16 + 1) * DB, NA = P::NDO < P::Rq ? P::NDO : P::Rq;
  static_assert(4 % DB == 0, "a wave's tiles must share one feature block");
  f32x4_t acc[NTR];
#pragma unroll
  for (int k = 0; k < NTR; ++k) acc[k] = accR[k];
#pragma unroll
  for (int s = 0; s < CH / 32; ++s) {
    Frag<NA> oa[NTR];
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int t = w + 4 * k < NRT ? w + 4 * k : w;  // past the grid (uneven split): a harmless repeat
      oa[k] = ot.template tfrag<NA>(32 * s, 16 * (t / DB), g, r16);
    }
    const Frag<P::Rq> qb = qt.template tfrag<P::Rq>(32 * s, 16 * (w % DB), g, r16);
    mmaf_tiles<NA, P::Rq>(acc, oa, qb);
  }
#pragma unroll
  for (int k = 0; k < NTR; ++k)
    if (w + 4 * k < NRT) accR[k] = acc[k];
}

// ===================================================================== B-A
// Feature slices (ns per value head, la_wide.h) see only their shares of
// den_i = phi(Q_i) . Z_i and of num_i . dO_i = phi(Q_i)^T S_i dO_i, so a wide
// head runs this pass twice:
//   kBqShares  the slice's two shares of token i go to gc[bh][i] (as a float2)
//              and nothing else is written;
//   kBqGiven   the pair (1/den_i, O_i . dO_i) of value head bh / ns, formed
//              from the sums of those shares, is read from gc instead of
//              recomputed and written.
// The pair is then exactly what a single head of all the features computes:
// the same states and products, summed over the slices.
constexpr int kBqFull = 0, kBqGiven = 1, kBqShares = 2;
template <typename T, int D, int M, int MODE = kBqFull>
__global__ __launch_bounds__(NT) void k_bq(const T* __restrict__ Q, const T* __restrict__ K,
                                            const T* __restrict__ V, const T* __restrict__ dO,
                                            const float* __restrict__ ckpt, T* __restrict__ dQ,
                                            float2* __restrict__ gc, float* __restrict__ ragg, int N, int L, int nseg,
                                            int fm, int ns) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NTS = DB * MB / 4;        // S^T tiles per wave
  constexpr int NRT = (MB + 1) * DB, NTR = (NRT + 3) / 4;  // [R | r]^T tiles: all, per wave (the last maybe short)
  static_assert((DB * MB) % 4 == 0, "S tiles must divide over four waves");
  __shared__ Planes<P::NQ, CH, D> qt;          // q' = phi(Q) / den, written by the query rows' own lanes
  __shared__ Planes<P::Ka, CH, D> kt;          // phi(K)
  __shared__ Planes<P::NV, CH, M> vt;          // V
  __shared__ Planes<P::NDO, CH, M + 16> ot;    // [dO | -O.dO | 0]
  __shared__ Planes<P::NS, D, M> sp;           // S before this chunk, [d][m]
  __shared__ alignas(16) float sZ[D];          // Z before this chunk

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int vh = MODE != kBqFull ? bh / ns : bh;  // value head
  const size_t offD = (size_t)bh * N * D, offM = (size_t)vh * N * M;
  const Frag<1> ones = ones_frag();
  ot.zero_cols(M + 2, M + 16);
  static_assert(4 % DB == 0, "a wave's S tiles must share one feature block");
  auto sdb = [&](int) { return w % DB; };  // (w + 4k) mod DB: the same for all of the wave's tiles
  auto smb = [&](int k) { return (w + 4 * k) / DB; };
  const bool zw = w < DB;  // holds Z of feature block w

  // the mask [j <= i] of the wave's query rows as B operands under the accumulator map (pairs of 16-row blocks)
  Frag<1> onef[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 32 * p + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
      onef[p].p[0][e] = j <= 16 * w + r16 ? (__bf16)1.0f : (__bf16)0.0f;
    }
  }

  const int nchunk = (t1 - t0 + CH - 1) / CH;
  // Q is needed only in the query rows' own lanes (row 16w + r16, features 16 d0 + 4g .. + 3, the layout of
  // U and Z_i), so each lane reads its elements straight into registers: phi(Q) is formed there in float32
  // and never staged (the q' rows written back below are all the LDS copy there is).
  typename IO<T>::raw4 qraw[DB];
  RowBuf<T, CH, D> bk;
  RowBuf<T, CH, M> bv, bd;
  auto fetch = [&](int c0) {
    const int nv = min(CH, t1 - c0);
    const int il = 16 * w + r16;
#pragma unroll
    for (int d0 = 0; d0 < DB; ++d0)
      qraw[d0] = il < nv ? IO<T>::load_raw4(Q + offD + (size_t)(c0 + il) * D + 16 * d0 + 4 * g) : IO<T>::zero_raw4();
    bk.load(K + offD + (size_t)c0 * D, nv);
    bv.load(V + offM + (size_t)c0 * M, nv);
    bd.load(dO + offM + (size_t)c0 * M, nv);
  };
  fetch(t0);

  // S^T tiles (acc[r] = S[16 db + r16][16 mb + 4 g + r]) and Z of block w, from the forward's checkpoint entry
  f32x4_t accS[NTS], accR[NTR];
  float zz = 0.f;
  {
    const float* st = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTS; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(st + (16 * sdb(k) + r16) * M + 16 * smb(k) + 4 * g);
      accS[k] = f32x4_t{a.x, a.y, a.z, a.w};
    }
    if (zw) zz = st[D * M + 16 * w + r16];
  }
#pragma unroll
  for (int k = 0; k < NTR; ++k) accR[k] = zero4();

  for (int ci = 0; ci < nchunk; ++ci) {
    const int c0 = t0 + ci * CH;
    const int nv = min(CH, t1 - c0);
    // ---- stage the state before this chunk and the chunk's operands (the barrier ending the previous
    // chunk separates them from every read of the previous ones)
    {
      float v4[4];
#pragma unroll
      for (int k = 0; k < NTS; ++k) {
        acc_to4(accS[k], v4);
        sp.put4(16 * sdb(k) + r16, 16 * smb(k) + 4 * g, v4);
      }
      if (zw && g == 0) sZ[16 * w + r16] = zz;
    }
    float qv[DB][4];  // phi(Q) of this lane's elements of its row (rows past the end: read as zero, unused)
#pragma unroll
    for (int d0 = 0; d0 < DB; ++d0) {
      IO<T>::unpack4(qraw[d0], qv[d0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[d0][r] = feat(qv[d0][r], fm);
    }
    bk.template stage_phi<P::Ka, CH, D, 8, 0>(kt, nv, nullptr, fm);
    bv.stage_values(vt);
    bd.stage_values(ot);
    if (ci + 1 < nchunk) fetch(c0 + CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);

    // ================ query rows il: S_i = S + sum_{j<=i} phi(K_j) V_j^T, Z_i likewise
    {
      const int il = 16 * w + r16;
      const bool row_ok = il < nv;
      constexpr int NO = cmax(P::Bt, P::U1_b);
      Frag<NO> dof[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) dof[s] = ot.template frag<NO>(il, 32 * s, g);
      // (V_j . dO_i) for j <= i as B operands under the accumulator map (pairs of 16-row blocks); blocks after
      // the wave's own stay zero.
      f32x4_t bt[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        bt[jb] = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mmaf<P::Bt, P::Bt>(bt[jb], vt.template frag<P::Bt>(16 * jb + r16, 32 * s, g), dof[s]);
        }
      }
      Frag<P::Ut> btf[2];
      // the wave's own block keeps j <= i (earlier blocks every pair, later ones are zero)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if (jb != w) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) bt[jb][r] = 4 * g + r <= r16 ? bt[jb][r] : 0.f;
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) btf[p] = acc2frag<P::Ut>(bt[2 * p], bt[2 * p + 1]);
      f32x4_t U[DB], ZC[DB];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) U[d0] = ZC[d0] = zero4();
      constexpr int NKA = P::Ka;
#pragma unroll
      for (int s = 0; s < M / 32; ++s) {
        Frag<P::U1_a> sa[DB];
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) sa[d0] = sp.template frag<P::U1_a>(16 * d0 + r16, 32 * s, g);
        mmaf_tiles<P::U1_a, P::U1_b>(U, sa, dof[s]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (2 * p <= w) {
          Frag<NKA> kfa[DB];
#pragma unroll
          for (int d0 = 0; d0 < DB; ++d0) kfa[d0] = kt.template tfrag_acc<NKA>(32 * p, 16 * d0, g, r16);
          mmaf_tiles<P::Ka, P::Ut>(U, kfa, btf[p]);
          mmaf_tiles<P::Ka, 1>(ZC, kfa, onef[p]);
        }
      }
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        const float4 z4 = *reinterpret_cast<const float4*>(&sZ[16 * d0 + 4 * g]);
        ZC[d0] += f32x4_t{z4.x, z4.y, z4.z, z4.w};  // U: S_i dO_i [d][i], ZC: Z_i [d][i]
      }
      float invz = 0.f, odo = 0.f;
      if constexpr (MODE == kBqGiven) {
        const float2 pr = row_ok ? gc[(size_t)vh * N + c0 + il] : make_float2(0.f, 0.f);
        invz = pr.x;
        odo = pr.y;
      } else {
        float pu = 0.f, pz = 0.f;
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pu += qv[d0][r] * U[d0][r];
            pz += qv[d0][r] * ZC[d0][r];
          }
        }
        pu = sum_over_g(pu);  // phi(Q_i)^T S_i dO_i = num_i . dO_i
        pz = sum_over_g(pz);  // phi(Q_i) . Z_i = den_i
        if constexpr (MODE == kBqShares) {
          if (g == 0 && row_ok) gc[(size_t)bh * N + c0 + il] = make_float2(pu, pz);
        } else {
          invz = row_ok ? 1.f / pz : 0.f;
          odo = row_ok ? pu * invz : 0.f;  // O_i . dO_i
        }
      }
      if constexpr (MODE != kBqShares) {
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
          float o[4], qs[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            o[r] = (U[d0][r] - ZC[d0][r] * odo) * invz * dfeat(qv[d0][r], fm);
            qs[r] = qv[d0][r] * invz;
          }
          if (row_ok) IO<T>::store4(dQ + offD + (size_t)(c0 + il) * D + 16 * d0 + 4 * g, o);
          qt.put4(il, 16 * d0 + 4 * g, qs);  // this lane's own elements of its own row: q'_i
        }
        if (g == 0) {
          if (MODE == kBqFull && row_ok) gc[(size_t)bh * N + c0 + il] = make_float2(invz, odo);
          put_neg_odo(ot, il, M, odo);
        }
      }
    }
    // (the shares pass writes nothing that the state update reads: no barrier)
    if constexpr (MODE != kBqShares) __syncthreads();

    // ================ the chunk's share of the reverse aggregate, then the state update
    if constexpr (MODE != kBqShares) rproduct64<T, D, M, NTR>(accR, ot, qt, w, g, r16);
    constexpr int NKB = P::Ka;
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      // phi(K)^T of the wave's feature block, read once for its S tiles and, where it holds Z, for Z
      const Frag<NKB> kb = kt.template tfrag<NKB>(32 * s, 16 * sdb(0), g, r16);
      Frag<P::dS_a> va[NTS];
#pragma unroll
      for (int k = 0; k < NTS; ++k) va[k] = vt.template tfrag<P::dS_a>(32 * s, 16 * smb(k), g, r16);
      mmaf_tiles<P::dS_a, P::Ka>(accS, va, kb);
      if (zw) {  // w < DB: its feature block is w
        f32x4_t dz = zero4();
        mmaf<1, P::Ka>(dz, ones, kb);
        zz += dz[0];
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  // the segment's reverse aggregate (sum over its tokens of phi(Q_i) g_i^T, c_i phi(Q_i)), [d][m] then r, for the
  // segments before it; segment 0's is not needed
  if (MODE != kBqShares && seg > 0) {
    float* out = ragg + ((size_t)bh * nseg + seg) * SV;
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
      if (t >= NRT) break;
      if (mb < MB) {
        *reinterpret_cast<float4*>(out + (16 * db + r16) * M + 16 * mb + 4 * g) =
            make_float4(accR[k][0], accR[k][1], accR[k][2], accR[k][3]);
      } else if (g == 0) {
        out[D * M + 16 * db + r16] = accR[k][0] + accR[k][1];  // rows M and M + 1 of the tile: r
      }
    }
  }
}

// ===================================================================== B-B
// Reverse walk of a segment: key rows form dK, dV from the reverse state
// after the chunk (R, r: the final-state gradient plus the later segments'
// aggregates plus the later chunks of this segment) and the chunk's own
// causal part; the same waves add the chunk's share to the reverse state in
// registers.  The sequence's first segment writes the reverse state carried
// through token 1: the gradient of the initial state (dS0, dZ0).
// PART (feature slices, ns per value head, la_wide.h): dV_j sums over all of
// a head's features, so each slice writes its share (float32, [bh][n][M] in
// pdv), summed over the slices afterwards.
template <typename T, int D, int M, bool PART = false>
__global__ __launch_bounds__(NT) void k_bkv(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, const T* __restrict__ dO,
                                             const float2* __restrict__ gc, const float* __restrict__ ragg,
                                             const float* __restrict__ dSN, const float* __restrict__ dZN,
                                             T* __restrict__ dK, T* __restrict__ dV, float* __restrict__ dS0,
                                             float* __restrict__ dZ0, int N, int L, int nseg, int scanned, int fm,
                                             int ns, float* __restrict__ pdv) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NRT = (MB + 1) * DB, NTR = (NRT + 3) / 4;  // [R | r]^T tiles: all, per wave (the last maybe short)
  __shared__ Planes<cmax(cmax(P::At, P::dK), P::Rq), CH, D> qt;  // q' = phi(Q) / den
  static_assert(P::NK >= cmax(P::At, P::Vk), "pass B's phi(K) products need their planes staged");
  __shared__ Planes<P::NK, CH, D> kt;          // phi(K)
  __shared__ Planes<P::NV, CH, M> vt;          // V
  __shared__ Planes<P::NDO, CH, M + 16> ot;    // [dO | -O.dO | 0]
  __shared__ Planes<P::NR, D, M> rp;           // R after this chunk, [d][m]
  __shared__ alignas(16) float sr[D];          // r after this chunk
  __shared__ alignas(16) float sOdo[CH];       // O_i . dO_i (0 past the end)

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int vh = PART ? bh / ns : bh;  // value head
  const size_t offD = (size_t)bh * N * D, offM = (size_t)vh * N * M;
  ot.zero_cols(M + 2, M + 16);

  const int nchunk = (t1 - t0 + CH - 1) / CH;
  using BQ = RowBuf<T, CH, D>;
  BQ bq;
  RowBuf<T, CH, D> bk;
  RowBuf<T, CH, M> bv, bd;
  float2 pgc = make_float2(0.f, 0.f);  // (1/den, O.dO) of token tid of the chunk (threads < CH)
  float pinv[BQ::CNT];                  // 1/den of the rows of this thread's Q vectors
  auto fetch = [&](int c0) {
    const int nv = min(CH, t1 - c0);
    bq.load(Q + offD + (size_t)c0 * D, nv);
    bk.load(K + offD + (size_t)c0 * D, nv);
    bv.load(V + offM + (size_t)c0 * M, nv);
    bd.load(dO + offM + (size_t)c0 * M, nv);
    if (tid < CH) pgc = tid < nv ? gc[(size_t)vh * N + c0 + tid] : make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < BQ::CNT; ++i) {
      const int row = BQ::row_of(i);
      pinv[i] = row < nv ? gc[(size_t)vh * N + c0 + row].x : 0.f;
    }
  };
  fetch(t0 + (nchunk - 1) * CH);

  // reverse state after the segment: the final-state gradient plus the later segments' aggregates (entry seg
  // of the suffix sums when scanned, which holds the sum over p > seg, else their sum in segment order),
  // summed through R's planes as scratch.  Tile k of wave w: t = w + 4k, value block t / DB (block MB: r),
  // feature block t % DB; acc[r] = R[16 db + r16][16 mb + 4 g + r].
  f32x4_t accR[NTR];
#pragma unroll
  for (int k = 0; k < NTR; ++k) accR[k] = zero4();
  const float* rg = nseg > 1 ? ragg + (size_t)bh * nseg * SV : nullptr;
  const bool later = rg && seg + 1 < nseg;
  if (later || dSN) {
    const int r0 = !later ? 0 : scanned ? seg : seg + 1, r1 = !later ? 0 : scanned ? seg + 1 : nseg;
    static_assert(sizeof(rp.v) >= SV * sizeof(float), "R planes too small to hold a float32 state");
    float* sbuf = reinterpret_cast<float*>(&rp.v[0][0][0]);
    sum_states<D, M, NT>(sbuf, dSN ? dSN + (size_t)bh * D * M : nullptr, dZN ? dZN + (size_t)bh * D : nullptr,
                         later ? rg : nullptr, r0, r1);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
      if (t >= NRT) break;
      if (mb < MB) {
        const float4 a = *reinterpret_cast<const float4*>(sbuf + (16 * db + r16) * M + 16 * mb + 4 * g);
        accR[k] = f32x4_t{a.x, a.y, a.z, a.w};
      } else if (g == 0) {
        accR[k][0] = sbuf[D * M + 16 * db + r16];  // r in row M of the tile
      }
    }
    __syncthreads();
  }

  for (int ci = nchunk - 1; ci >= 0; --ci) {
    const int c0 = t0 + ci * CH;
    const int nv = min(CH, t1 - c0);
    // ---- stage R, r after this chunk and the chunk's operands
    {
      float v4[4];
#pragma unroll
      for (int k = 0; k < NTR; ++k) {
        const int t = w + 4 * k, mb = t / DB, db = t % DB;
        if (t >= NRT) break;
        if (mb < MB) {
          acc_to4(accR[k], v4);
          rp.put4(16 * db + r16, 16 * mb + 4 * g, v4);
        } else if (g == 0) {
          sr[16 * db + r16] = accR[k][0] + accR[k][1];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < BQ::CNT; ++i) {  // q' = phi(Q) / den from this thread's Q vectors
      float x[BQ::E];
      IO<T>::unpack(bq.r[i], x);
#pragma unroll
      for (int e = 0; e < BQ::E; ++e) x[e] = feat(x[e], fm) * pinv[i];
      qt.template put<BQ::E>(BQ::row_of(i), BQ::col_of(i), x);
    }
    bk.template stage_phi<P::NK, CH, D, 8, 0>(kt, nv, nullptr, fm);
    bv.stage_values(vt);
    bd.stage_values(ot);
    if (tid < CH) {
      sOdo[tid] = pgc.y;
      put_neg_odo(ot, tid, M, pgc.y);
    }
    if (ci > 0) fetch(c0 - CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);

    // ================ key rows jl
    {
      constexpr int NKT = cmax(P::At, P::Vk);
      constexpr int NVT = cmax(P::Wt, P::KR_b);
      const int jl = 16 * w + r16;
      const bool row_ok = jl < nv;
      Frag<NKT> kfr[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kfr[s] = kt.template frag<NKT>(jl, 32 * s, g);
      Frag<NVT> vfr[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) vfr[s] = vt.template frag<NVT>(jl, 32 * s, g);
      // A'_ij = q'_i . phi(K_j) and W'_ij = dO_i . V_j - O_i . dO_i (rows i, columns j), zero where i < j (whole
      // blocks before this wave's, and the upper triangle of its own), in pairs of 16-row blocks as B operands
      // under the accumulator map.
      f32x4_t at[4], wt[4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        at[ib] = wt[ib] = zero4();
        if (ib >= w) {
#pragma unroll
          for (int s = 0; s < D / 32; ++s)
            mmaf<P::At, P::At>(at[ib], qt.template frag<P::At>(16 * ib + r16, 32 * s, g), kfr[s]);
#pragma unroll
          for (int s = 0; s < M / 32; ++s)
            mmaf<P::Wt, P::Wt>(wt[ib], ot.template frag<P::Wt>(16 * ib + r16, 32 * s, g), vfr[s]);
        }
      }
      // blocks before the wave's own stay zero; later blocks keep every pair; the wave's own keeps i >= j
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        if (ib < w) continue;
        const float4 od = *reinterpret_cast<const float4*>(&sOdo[16 * ib + 4 * g]);
        const float odr[4] = {od.x, od.y, od.z, od.w};
        if (ib > w) {
#pragma unroll
          for (int r = 0; r < 4; ++r) wt[ib][r] -= odr[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool keep = 4 * g + r >= r16;
            at[ib][r] = keep ? at[ib][r] : 0.f;
            wt[ib][r] = keep ? wt[ib][r] - odr[r] : 0.f;
          }
        }
      }
      Frag<P::dK> wfr[2];
      Frag<P::dV> afr[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        wfr[p] = acc2frag<P::dK>(wt[2 * p], wt[2 * p + 1]);
        afr[p] = acc2frag<P::dV>(at[2 * p], at[2 * p + 1]);
      }
      // dK_j = (R V_j + r + sum_{i>=j} q'_i W'_ij) phi'(K_j), the feature blocks' tiles together
      f32x4_t aK[DB];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) aK[d0] = zero4();
#pragma unroll
      for (int s = 0; s < M / 32; ++s) {
        Frag<P::KR_a> ra[DB];
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) ra[d0] = rp.template frag<P::KR_a>(16 * d0 + r16, 32 * s, g);
        mmaf_tiles<P::KR_a, P::KR_b>(aK, ra, vfr[s]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (2 * p + 1 >= w) {
          Frag<P::dK> qa[DB];
#pragma unroll
          for (int d0 = 0; d0 < DB; ++d0) qa[d0] = qt.template tfrag_acc<P::dK>(32 * p, 16 * d0, g, r16);
          mmaf_tiles<P::dK, P::dK>(aK, qa, wfr[p]);
        }
      }
      if (row_ok) {
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
          float o[4], kv[4];
          kt.get4(jl, 16 * d0 + 4 * g, kv);
          const float4 r4 = *reinterpret_cast<const float4*>(&sr[16 * d0 + 4 * g]);
          const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (aK[d0][r] + rr[r]) * dfeat(kv[r], fm);
          IO<T>::store4(dK + offD + (size_t)(c0 + jl) * D + 16 * d0 + 4 * g, o);
        }
      }
      // dV_j = R^T phi(K_j) + sum_{i>=j} dO_i A'_ij, the value blocks' tiles together
      constexpr int NA = P::NDO < P::dV ? P::NDO : P::dV;
      f32x4_t aV[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) aV[mb] = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        Frag<P::VR> ra[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) ra[mb] = rp.template tfrag<P::VR>(32 * s, 16 * mb, g, r16);
        mmaf_tiles<P::VR, P::Vk>(aV, ra, kfr[s]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (2 * p + 1 >= w) {
          Frag<NA> oa[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) oa[mb] = ot.template tfrag_acc<NA>(32 * p, 16 * mb, g, r16);
          mmaf_tiles<NA, P::dV>(aV, oa, afr[p]);
        }
      }
      if (row_ok) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if constexpr (PART) {
            *reinterpret_cast<float4*>(pdv + ((size_t)bh * N + c0 + jl) * M + 16 * mb + 4 * g) =
                make_float4(aV[mb][0], aV[mb][1], aV[mb][2], aV[mb][3]);
          } else {
            float o[4] = {aV[mb][0], aV[mb][1], aV[mb][2], aV[mb][3]};
            IO<T>::store4(dV + offM + (size_t)(c0 + jl) * M + 16 * mb + 4 * g, o);
          }
        }
      }
    }
    // ================ the chunk's share of the reverse state (for the earlier chunks)
    rproduct64<T, D, M, NTR>(accR, ot, qt, w, g, r16);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  // the reverse state carried through the sequence's first token is the gradient of the initial state
  if (t0 == 0 && dS0) {
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int t = w + 4 * k, mb = t / DB, db = t % DB;
      if (t >= NRT) break;
      if (mb < MB) {
        *reinterpret_cast<float4*>(dS0 + (size_t)bh * D * M + (16 * db + r16) * M + 16 * mb + 4 * g) =
            make_float4(accR[k][0], accR[k][1], accR[k][2], accR[k][3]);
      } else if (g == 0) {
        dZ0[(size_t)bh * D + 16 * db + r16] = accR[k][0] + accR[k][1];
      }
    }
  }
}

}  // namespace la
