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
// non-causal backward also the reverse totals (R, r) -- in registers, with the chunk's
// operands staged once per chunk in LDS, token-major, as bf16 planes
// (la_device.h) while the next chunk's global reads are in flight.  A
// segment's start state is the sum, in a fixed order, of the aggregates of
// the segments before it (after it, for the reverse state), written by a
// separate aggregate pass: results are bitwise reproducible and no workgroup
// waits for another.
//
// Wave priority.  Two workgroups share each compute unit, so every SIMD runs
// two wavefronts that are usually in different phases of their chunks.  A
// wavefront raises its priority for the compute phase of a chunk (after the
// staging barrier) and lowers it for staging, so the matrix and vector work of
// one interleaves with the other's loads and LDS stores (measured on the
// 2^16-token workload: forward 129 -> 121.5 us; the backward passes, which do
// the same in la_bwd2.h, 232 -> 227 and 211 -> 203 us).
//
// Inside a chunk every contraction is a 16x16 MFMA tile product; wave w owns
// the 16 tokens 16w..16w+15 of a 64-token chunk.  Sums over tokens of a single
// vector (the normaliser Z, the reverse normaliser r) are MFMA products with
// an all-ones operand, the form of eq. 14-15 on [V, 1].
#pragma once

#include "la_device.h"

namespace la {

constexpr int CH = 64;  // forward chunk

// Workgroup -> item = head * nseg + segment, for the kernels launched with
// one workgroup per segment (grid = heads x nseg).  Workgroups go to the
// eight XCDs round-robin (workgroup i to XCD i mod 8), each XCD with its own
// L2.  When every XCD's share is a whole number of heads, the workgroups of
// one XCD take whole heads: the segments of a head, which read one another's
// aggregates and checkpoint entries kernel after kernel, then meet in one L2,
// and within a head a lower segment keeps a lower workgroup index.  Otherwise
// the items follow the workgroup index.
__device__ __forceinline__ int seg_item(int nseg) {
  constexpr int NX = 8;
  const int nb = (int)gridDim.x, i = (int)blockIdx.x;
  if (nb % NX != 0 || (nb / NX) % nseg != 0) return i;
  return (i % NX) * (nb / NX) + i / NX;
}

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
  // forward: phi(Q), phi(K) in A^T, phi(K) in the state update, V, S^T, A,
  // Z (the denominator is an output, and a 1-plane Z would leave it at bf16
  // accuracy; two planes keep it near float32)
  static constexpr int FQ = 1, FK = 1, FKF = 2, FV = 1, FS = 1, FA = 1, FZ = 2;
  // backward staging (la_bwd2.h and the non-causal backward): phi(Q), phi(K)
  // in pass B (its products take one plane; the staged value also gives
  // phi'(K) = min(phi, 1) to the bf16 dK, which one plane carries to bf16
  // accuracy), V, dO, [g | c], S, R
  static constexpr int NQ = 2, NK = 1, NV = 1, NDO = 1, NG = 2, NS = 2, NR = 2;
  // backward products: the non-causal backward's, and in the two-pass causal
  // backward V^T phi(K) (dS_a), dO.V (Bt, Wt), S dO (U1) and R V (KR)
  static constexpr int dS_a = 1, Bt = 1, U1_a = 2, U1_b = 1, dR = 2, Wt = 1, KR_a = 2, KR_b = 1, VR = 2;
  // the two-pass causal backward's other products: phi(K) in pass A's chunk
  // products and S, Z update (Ka), the masked V.dO there (Ut), q' in the
  // reverse aggregates of both passes (Rq) -- all three feed running sums or
  // the cancellations of eq. 13-14, where phi(x) ~ 1 + x leaves the rounding
  // of a one-plane phi near 2^-9 against deviations of size x, so they keep
  // two planes -- and pass B's q'.phi(K) (At), q'^T W' (dK), dO A' (dV) and
  // the phi(K) of R^T phi(K) (Vk; R keeps VR planes): per-term products
  // within a chunk or against a two-plane state, one plane.
  static constexpr int Ka = 2, Ut = 2, Rq = 2, At = 1, dK = 2, dV = 1, Vk = 1;
};
template <>
struct Prec<float> {
  static constexpr int FQ = 2, FK = 2, FKF = 3, FV = 3, FS = 2, FA = 2, FZ = 2;
  static constexpr int NQ = 3, NK = 2, NV = 3, NDO = 3, NG = 2, NS = 3, NR = 2;
  // g_i.V_j - O_i.dO_i cancels where V_j = O_i, so dO.V and its product with
  // phi(Q) are taken at float32 level too (bf16 inputs make dO.V exact).
  static constexpr int dS_a = 3, Bt = 3, U1_a = 3, U1_b = 3, dR = 2, Wt = 3, KR_a = 2, KR_b = 2, VR = 2;
  static constexpr int Ka = 3, Ut = 3, Rq = 2, At = 2, dK = 3, dV = 2, Vk = 2;
};

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// State tiles.  Tile t = w + 4k of wave w covers feature block db = t % DB
// (the same for all of the wave's tiles, since DB divides 4) and value block
// mb = t / DB.  Two register layouts are used:
//   S layout:  acc[k][r] = S[16db + 4g + r][16mb + r16]
//   S^T layout: acc[k][r] = S[16db + r16][16mb + 4g + r]
// for a row-major D x M state S in global memory.
template <int D, int M, int NTW>
__device__ __forceinline__ void add_S_tiles(f32x4_t* acc, const float* base, long stride, int p0, int p1, int w,
                                            int r16, int g) {
  constexpr int DB = D / 16;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    const float* e = base + (16 * db + 4 * g) * M + 16 * mb + r16;
    for (int p = p0; p < p1; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[k][r] += e[(long)p * stride + r * M];
  }
}
template <int D, int M, int NTW>
__device__ __forceinline__ void store_S_tiles(float* dst, const f32x4_t* acc, int w, int r16, int g) {
  constexpr int DB = D / 16;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    float* e = dst + (16 * db + 4 * g) * M + 16 * mb + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r * M] = acc[k][r];
  }
}
template <int D, int M, int NTW>
__device__ __forceinline__ void add_ST_tiles(f32x4_t* acc, const float* base, long stride, int p0, int p1, int w,
                                             int r16, int g) {
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
template <int D, int M, int NTW>
__device__ __forceinline__ void store_ST_tiles(float* dst, const f32x4_t* acc, int w, int r16, int g) {
  constexpr int DB = D / 16;
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int t = w + 4 * k, mb = t / DB, db = t % DB;
    *reinterpret_cast<float4*>(dst + (16 * db + r16) * M + 16 * mb + 4 * g) =
        make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
}

// sb[e] = init[e] + sum over p in [p0, p1), in order, of base[p * SV + e] for
// the D*M + D floats of a state (S then Z; init from S0/Z0 or zero).  The
// whole workgroup sums: each thread owns float4 columns and keeps a batch of
// 16 independent loads in flight.  The caller synchronises before reading sb.
template <int D, int M, int NTH = NT>
__device__ __forceinline__ void sum_states(float* sb, const float* S0, const float* Z0, const float* base, int p0,
                                           int p1) {
  constexpr int SV = D * M + D, BT = 16;
  for (int e = 4 * threadIdx.x; e < SV; e += 4 * NTH) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* init = e < D * M ? (S0 ? S0 + e : nullptr) : (Z0 ? Z0 + (e - D * M) : nullptr);
    if (init) acc = *reinterpret_cast<const float4*>(init);
    for (int p = p0; p < p1; p += BT) {
      float4 v[BT];
#pragma unroll
      for (int j = 0; j < BT; ++j)
        v[j] = p + j < p1 ? *reinterpret_cast<const float4*>(base + (size_t)(p + j) * SV + e)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < BT; ++j) {
        acc.x += v[j].x;
        acc.y += v[j].y;
        acc.z += v[j].z;
        acc.w += v[j].w;
      }
    }
    *reinterpret_cast<float4*>(sb + e) = acc;
  }
}

__device__ __forceinline__ void acc_to4(const f32x4_t& a, float* o) {
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
}

// ===================================================================== F1
// Segment aggregates: agg[bh][seg] = ( sum_j phi(K_j) V_j^T  [D][M],
//                                      sum_j phi(K_j)        [D] )
// over the segment's tokens (eq. 10-11 restricted to one segment).  With ns
// > 1 the heads are feature slices: head bh holds features of value head
// bh / ns (wide feature maps, la_wide.h).
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_seg_state(const T* __restrict__ K, const T* __restrict__ V,
                                                   float* __restrict__ agg, int N, int L, int nseg, int fm, int ns) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  __shared__ Planes<P::FKF, CH, D> kt;
  __shared__ Planes<P::FV, CH, M> vt;

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)(bh / ns) * N * M;
  const Frag<1> ones = ones_frag();

  f32x4_t acc[NTW], accZ = zero4();  // S layout; accZ[r] = Z[16db + 4g + r]
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();

  // two chunks of global reads in flight: the buffer of a chunk is refilled
  // with the chunk two ahead as soon as it has been staged
  RowBuf<T, CH, D> bk[2];
  RowBuf<T, CH, M> bv[2];
  auto fetch = [&](RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      k_.load(Kh + (size_t)c0 * D, nv);
      v_.load(Vh + (size_t)c0 * M, nv);
    }
  };
  auto chunk = [&](RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    k_.stage_phi(kt, nv, nullptr, fm);
    v_.stage_values(vt);
    fetch(k_, v_, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      const Frag<P::FKF> ka = kt.template tfrag<P::FKF>(32 * s, 16 * db, g, r16);
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int mb = (w + 4 * k) / DB;
        mmaf<P::FKF, P::FV>(acc[k], ka, vt.template tfrag<P::FV>(32 * s, 16 * mb, g, r16));
      }
      if (zw) mmaf<P::FKF, 1>(accZ, ka, ones);
    }
  };
  fetch(bk[0], bv[0], t0);
  fetch(bk[1], bv[1], t0 + CH);
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(bk[0], bv[0], c0);
    if (c0 + CH < t1) chunk(bk[1], bv[1], c0 + CH);
  }
  float* out = agg + ((size_t)bh * nseg + seg) * SV;
  store_S_tiles<D, M, NTW>(out, acc, w, r16, g);
  if (zw && r16 == 0)
    *reinterpret_cast<float4*>(out + D * M + 16 * db + 4 * g) = make_float4(accZ[0], accZ[1], accZ[2], accZ[3]);
}

// ===================================================================== F3
// Chunked forward over one segment.
//   causal: for each chunk, A^T = phi(K) phi(Q)^T masked to j <= i (eq. 8),
//     num^T = V^T A^T + S^T phi(Q)^T and den = rowsum(A) + phi(Q) Z,
//     O = num / den (eq. 9-12), then S += phi(K)^T V, Z += phi(K)^T 1
//     (eq. 10-11).  The start state is entry seg of the prefix states `pref`
//     ([bh][nseg + 1][S | Z], written by k_scan_states) when given, else
//     (S0, Z0) plus the aggregates `agg` of the earlier segments, summed in
//     segment order here; in that case the start state goes to checkpoint
//     entry seg and the last segment writes entry nseg.  The last segment
//     writes the final state to S_out/Z_out.
//   non-causal: num^T = S^T phi(Q)^T, den = Z^T phi(Q)^T with S, Z the total:
//     entry nseg of `pref`, or the sum of all aggregates (eq. 5-6); segment 0
//     writes the total to S_out/Z_out when given.
// Z is staged as 16 identical rows, so phi(Q) Z is one more MFMA output tile
// whose every row holds the denominators of the wave's tokens.
// PART (feature slices, ns per value head, la_wide.h): the slice's share of
// the numerator (float32, [bh][n][M] in pnum) and of the denominator (den_out)
// instead of O; they are summed over the slices afterwards.
template <typename T, int D, int M, bool CAUSAL, bool PART = false>
__global__ __launch_bounds__(NT) void k_fwd(const T* __restrict__ Q, const T* __restrict__ K,
                                             const T* __restrict__ V, T* __restrict__ O, float* __restrict__ den_out,
                                             const float* __restrict__ pref, const float* __restrict__ agg,
                                             const float* __restrict__ S0, const float* __restrict__ Z0,
                                             float* __restrict__ ckpt,
                                             float* __restrict__ S_out, float* __restrict__ Z_out, int N, int L,
                                             int nseg, int fm, int ns, float* __restrict__ pnum) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D;
  constexpr int KR = CAUSAL ? CH : 1, KD = CAUSAL ? D : 8, KM = CAUSAL ? M : 8;
  using KPlanes = Planes<P::FKF, KR, KD>;
  constexpr size_t KB_ = sizeof(KPlanes), SB_ = (size_t)SV * sizeof(float);
  __shared__ Planes<P::FQ, CH, D> qt;
  __shared__ Planes<P::FV, KR, KM> vt;
  __shared__ Planes<P::FS, M, D> st;       // S^T
  __shared__ Planes<P::FZ, 16, D> zr;      // 16 copies of Z
  // The start state is summed in LDS and read into registers before the first
  // chunk is staged (a barrier lies between), so in the causal kernel its
  // buffer shares storage with the phi(K) planes: 8 KB less at D = 64, M = 32
  // float32 (two workgroups per compute unit instead of one), 16 KB less at
  // D = M = 64 bf16 (three instead of two).
  __shared__ alignas(16) unsigned char kmem[CAUSAL && SB_ > KB_ ? SB_ : KB_];
  __shared__ alignas(16) float sown[CAUSAL ? 4 : SV];
  KPlanes& kt = *reinterpret_cast<KPlanes*>(kmem);
  float* const sbuf = CAUSAL ? reinterpret_cast<float*>(kmem) : sown;  // start state summed from the aggregates

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)(PART ? bh / ns : bh) * N * M;
  T* Oh = PART ? nullptr : O + (size_t)bh * N * M;
  float* Ph = PART ? pnum + (size_t)bh * N * M : nullptr;
  const Frag<1> ones = ones_frag();

  // two chunks of global reads in flight (see k_seg_state)
  RowBuf<T, CH, D> bq[2], bk[2];
  RowBuf<T, CH, M> bv[2];
  auto fetch = [&](RowBuf<T, CH, D>& q_, RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      q_.load(Qh + (size_t)c0 * D, nv);
      if constexpr (CAUSAL) {
        k_.load(Kh + (size_t)c0 * D, nv);
        v_.load(Vh + (size_t)c0 * M, nv);
      }
    }
  };
  fetch(bq[0], bk[0], bv[0], t0);
  fetch(bq[1], bk[1], bv[1], t0 + CH);

  // ---- start state (S layout), Z for the wave's feature block
  f32x4_t accS[NTW], accZ = zero4();
#pragma unroll
  for (int k = 0; k < NTW; ++k) accS[k] = zero4();
  if (pref) {
    const float* st0 = pref + ((size_t)bh * (nseg + 1) + (CAUSAL ? seg : nseg)) * SV;
    add_S_tiles<D, M, NTW>(accS, st0, 0, 0, 1, w, r16, g);
    if (zw) {
      const float4 z4 = *reinterpret_cast<const float4*>(st0 + D * M + 16 * db + 4 * g);
      accZ = f32x4_t{z4.x, z4.y, z4.z, z4.w};
    }
  } else {
    const int pend = agg ? (CAUSAL ? seg : nseg) : 0;
    sum_states<D, M>(sbuf, S0 ? S0 + (size_t)bh * D * M : nullptr, Z0 ? Z0 + (size_t)bh * D : nullptr,
                     agg ? agg + (size_t)bh * nseg * SV : nullptr, 0, pend);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int mb = (w + 4 * k) / DB;
#pragma unroll
      for (int r = 0; r < 4; ++r) accS[k][r] = sbuf[(16 * db + 4 * g + r) * M + 16 * mb + r16];
    }
    if (zw) {
#pragma unroll
      for (int r = 0; r < 4; ++r) accZ[r] = sbuf[D * M + 16 * db + 4 * g + r];
    }
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
  if (CAUSAL && ckpt) {
    float* ck = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
    write_state(ck, ck + D * M);
  }
  if (!CAUSAL && S_out && seg == 0) write_state(S_out + (size_t)bh * D * M, Z_out + (size_t)bh * D);
  stage_state();

  auto chunk = [&](RowBuf<T, CH, D>& q_, RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    q_.stage_phi(qt, nv, nullptr, fm);
    if constexpr (CAUSAL) {
      k_.stage_phi(kt, nv, nullptr, fm);
      v_.stage_values(vt);
    }
    fetch(q_, k_, v_, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);

    const int il = 16 * w + r16;
    Frag<P::FQ> qf[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = qt.template frag<P::FQ>(il, 32 * s, g);

    Frag<P::FA> af[2];
    float dp = 0.f;  // row sum of the masked A, float32
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
      dp = sum_over_g(dp);
    }
    f32x4_t dn = zero4();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) mmaf<P::FZ, P::FQ>(dn, zr.template frag<P::FZ>(r16, 32 * s, g), qf[s]);
    const float den = dp + dn[0];  // every row of the Z tile holds phi(Q_i).Z, i = il
    const float inv = 1.f / den;
    const bool row_ok = il < nv;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t acc = zero4();
      if constexpr (CAUSAL) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p <= w) mmaf<P::FV, P::FA>(acc, vt.template tfrag_acc<P::FV>(32 * p, 16 * mb, g, r16), af[p]);
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mmaf<P::FS, P::FQ>(acc, st.template frag<P::FS>(16 * mb + r16, 32 * s, g), qf[s]);
      if (row_ok) {
        if constexpr (PART) {
          *reinterpret_cast<float4*>(Ph + (size_t)(c0 + il) * M + 16 * mb + 4 * g) =
              make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = acc[r] * inv;
          IO<T>::store4(Oh + (size_t)(c0 + il) * M + 16 * mb + 4 * g, o);
        }
      }
    }
    if (den_out && g == 0 && row_ok) den_out[(size_t)bh * N + c0 + il] = den;

    if constexpr (CAUSAL) {
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const Frag<P::FKF> ka = kt.template tfrag<P::FKF>(32 * s, 16 * db, g, r16);
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          const int mb = (w + 4 * k) / DB;
          mmaf<P::FKF, P::FV>(accS[k], ka, vt.template tfrag<P::FV>(32 * s, 16 * mb, g, r16));
        }
        if (zw) mmaf<P::FKF, 1>(accZ, ka, ones);
      }
      __syncthreads();
      stage_state();
    }
  };
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(bq[0], bk[0], bv[0], c0);
    if (c0 + CH < t1) chunk(bq[1], bk[1], bv[1], c0 + CH);
  }
  if constexpr (CAUSAL) {
    if (seg == nseg - 1) {
      if (ckpt) {
        float* ck = ckpt + ((size_t)bh * (nseg + 1) + nseg) * SV;
        write_state(ck, ck + D * M);
      }
      if (S_out) write_state(S_out + (size_t)bh * D * M, Z_out + (size_t)bh * D);
    }
  }
}

// ===================================================================== F4
// Causal forward in one launch, for segments of at most NC chunks: the
// aggregate pass of F1 is folded in by deferring each segment's carry.
//
// Workgroup b owns segment b % nseg of head b / nseg and waits only for the
// lower-numbered workgroups of its head.  Workgroups are dispatched in order
// of their index on each XCD, so the lowest unfinished workgroup is always
// resident and never waits: the waits end.  (A ticket taken from a counter at
// workgroup start would not depend on that order, but same-address atomics
// from every workgroup serialise: measured 0.11 us per workgroup.)  The
// workgroup walks its segment from a zero state exactly as F3 does, but
// keeps, per chunk, the unnormalised numerators V^T A^T + S_loc^T phi(Q)^T,
// the denominators
// rowsum(A) + phi(Q).Z_loc and the phi(Q) fragments in registers instead of
// writing O.  At the end (S_loc, Z_loc) is the segment aggregate (eq. 10-11
// over the segment): it is published with a flag, the aggregates of the
// earlier segments of the head are summed in segment order onto (S0, Z0) into
// the carry (S_c, Z_c), and O = (num + S_c^T phi(Q)) / (den + phi(Q).Z_c),
// since by eq. 12 the state seen by token i is S_c plus the segment's tokens
// up to i.  Checkpoint entries and the final state are written as by F3.
//
// sync: [0] error flag, [1 + bh * nseg + seg] published flag; all zero at
// launch.  Each wait is bounded: a workgroup that polls too long sets the
// error flag, makes its carry NaN (so that its rows of O, den and the states
// it writes show the failure instead of a wrong value) and goes on, so every
// wave reaches the end of the kernel.
//
// Coherence between XCDs.  Each XCD has its own L2, so data passed between
// workgroups must not sit in (or be read from) one of them.  The aggregates
// and flags are therefore written and read only with relaxed atomics of
// device ("agent") scope, which write through and read past the L2; the
// aggregate stores are complete (waited for) before the barrier that
// precedes the flag store, and the aggregate loads are issued after the
// barrier that follows the flag load.  Release and acquire fences of device
// scope would instead write back and invalidate the whole L2 of the XCD for
// every workgroup (measured: 24 -> 119 us on the MNIST-shaped layer).

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<unsigned*>(const_cast<float*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// true when the flag was seen set within `polls` polls (polls = 0: gives up
// at once without looking).  A wait that gives up sets the status word err
// and, when given, the caller's status word xerr.
__device__ __forceinline__ bool lb_wait(const unsigned* f, unsigned* err, unsigned* xerr, int polls) {
  for (int it = 0; it < polls; ++it) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  if (polls > 0 && __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return true;
  atomicOr(err, 1u);
  if (xerr) atomicOr(xerr, 1u);
  return false;
}

template <typename T, int D, int M, int NC>
__global__ __launch_bounds__(NT) void k_fwd_lb(const T* __restrict__ Q, const T* __restrict__ K,
                                                const T* __restrict__ V, T* __restrict__ O,
                                                float* __restrict__ den_out, const float* __restrict__ S0,
                                                const float* __restrict__ Z0, float* __restrict__ agg,
                                                unsigned* __restrict__ sync, float* __restrict__ ckpt,
                                                float* __restrict__ S_out, float* __restrict__ Z_out, int N, int L,
                                                int nseg, int fm, int polls, unsigned* __restrict__ xstatus) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, NTW = DB * MB / 4, SV = D * M + D, DS = D / 32;
  using KPlanes = Planes<P::FKF, CH, D>;
  constexpr size_t KB_ = sizeof(KPlanes), SB_ = (size_t)SV * sizeof(float);
  __shared__ Planes<P::FQ, CH, D> qt;
  __shared__ Planes<P::FV, CH, M> vt;
  __shared__ Planes<P::FS, M, D> st;   // S^T: the segment's running state, then the carry
  __shared__ Planes<P::FZ, 16, D> zr;  // 16 copies of Z
  // phi(K) planes during the walk; the carry summed from the aggregates after it
  __shared__ alignas(16) unsigned char kmem[SB_ > KB_ ? SB_ : KB_];
  KPlanes& kt = *reinterpret_cast<KPlanes*>(kmem);
  float* const sbuf = reinterpret_cast<float*>(kmem);

  const int item = seg_item(nseg);
  const int seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * M;
  T* Oh = O + (size_t)bh * N * M;
  const Frag<1> ones = ones_frag();

  RowBuf<T, CH, D> bq[2], bk[2];
  RowBuf<T, CH, M> bv[2];
  auto fetch = [&](RowBuf<T, CH, D>& q_, RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      q_.load(Qh + (size_t)c0 * D, nv);
      k_.load(Kh + (size_t)c0 * D, nv);
      v_.load(Vh + (size_t)c0 * M, nv);
    }
  };
  fetch(bq[0], bk[0], bv[0], t0);
  fetch(bq[1], bk[1], bv[1], t0 + CH);

  // segment state from zero (S layout); staged as S^T planes and Z rows
  f32x4_t accS[NTW], accZ = zero4();
#pragma unroll
  for (int k = 0; k < NTW; ++k) accS[k] = zero4();
  auto stage = [&](const f32x4_t* s_, const f32x4_t& z_) {
    float v4[4];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      acc_to4(s_[k], v4);
      st.put4(16 * ((w + 4 * k) / DB) + r16, 16 * db + 4 * g, v4);
    }
    if (zw) {
      acc_to4(z_, v4);
      zr.put4(r16, 16 * db + 4 * g, v4);
    }
  };
  stage(accS, accZ);

  // per chunk: numerators (O^T tiles), denominators and phi(Q) fragments
  f32x4_t num[NC][MB];
  float dl[NC];
  Frag<P::FQ> qk[NC][DS];

#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int c0 = t0 + c * CH;
    if (c0 < t1) {
      RowBuf<T, CH, D>& q_ = bq[c & 1];
      RowBuf<T, CH, D>& k_ = bk[c & 1];
      RowBuf<T, CH, M>& v_ = bv[c & 1];
      const int nv = min(CH, t1 - c0);
      __syncthreads();
      q_.stage_phi(qt, nv, nullptr, fm);
      k_.stage_phi(kt, nv, nullptr, fm);
      v_.stage_values(vt);
      if (c + 2 < NC) fetch(q_, k_, v_, c0 + 2 * CH);
      __syncthreads();

      const int il = 16 * w + r16;
#pragma unroll
      for (int s = 0; s < DS; ++s) qk[c][s] = qt.template frag<P::FQ>(il, 32 * s, g);

      f32x4_t accA[4];
      float dp = 0.f;  // row sum of the masked A, float32
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4_t a = zero4();
        if (jb <= w) {
#pragma unroll
          for (int s = 0; s < DS; ++s)
            mmaf<P::FK, P::FQ>(a, kt.template frag<P::FK>(16 * jb + r16, 32 * s, g), qk[c][s]);
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
      Frag<P::FA> af[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) af[p] = acc2frag<P::FA>(accA[2 * p], accA[2 * p + 1]);
      dp = sum_over_g(dp);
      f32x4_t dn = zero4();
#pragma unroll
      for (int s = 0; s < DS; ++s) mmaf<P::FZ, P::FQ>(dn, zr.template frag<P::FZ>(r16, 32 * s, g), qk[c][s]);
      dl[c] = dp + dn[0];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (2 * p <= w) mmaf<P::FV, P::FA>(acc, vt.template tfrag_acc<P::FV>(32 * p, 16 * mb, g, r16), af[p]);
#pragma unroll
        for (int s = 0; s < DS; ++s)
          mmaf<P::FS, P::FQ>(acc, st.template frag<P::FS>(16 * mb + r16, 32 * s, g), qk[c][s]);
        num[c][mb] = acc;
      }
      // S += phi(K)^T V, Z += phi(K)^T 1 (eq. 10-11)
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const Frag<P::FKF> ka = kt.template tfrag<P::FKF>(32 * s, 16 * db, g, r16);
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          const int mb = (w + 4 * k) / DB;
          mmaf<P::FKF, P::FV>(accS[k], ka, vt.template tfrag<P::FV>(32 * s, 16 * mb, g, r16));
        }
        if (zw) mmaf<P::FKF, 1>(accZ, ka, ones);
      }
      if (c0 + CH < t1) {
        __syncthreads();
        stage(accS, accZ);
      }
    }
  }

  // publish the segment aggregate (the last segment has no successor)
  if (seg + 1 < nseg) {
    float* ag = agg + (size_t)item * SV;
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int t = w + 4 * k, mb = t / DB;
      float* e = ag + (16 * db + 4 * g) * M + 16 * mb + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) st_dev(e + r * M, accS[k][r]);
    }
    if (zw && r16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st_dev(ag + D * M + 16 * db + 4 * g + r, accZ[r]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);  // every aggregate store acknowledged
  }
  __syncthreads();  // aggregate written; phi(K) planes, st and zr no longer read
  if (seg + 1 < nseg && tid == 0) __hip_atomic_store(&sync[1 + item], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // carry: (S0, Z0) plus the earlier segments' aggregates, in segment order
  bool late = false;
  for (int p = tid; p < seg; p += NT) late |= !lb_wait(&sync[1 + (size_t)bh * nseg + p], &sync[0], xstatus, polls);
  const bool failed = __syncthreads_or(late);
  {
    const float* a0 = agg + (size_t)bh * nseg * SV;
    const float* s0h = S0 ? S0 + (size_t)bh * D * M : nullptr;
    const float* z0h = Z0 ? Z0 + (size_t)bh * D : nullptr;
    constexpr int BT = 8;
    for (int e = tid; e < SV; e += NT) {
      float acc = 0.f;
      if (e < D * M) {
        if (s0h) acc = s0h[e];
      } else if (z0h) {
        acc = z0h[e - D * M];
      }
      for (int p = 0; p < seg; p += BT) {
        float v[BT];
#pragma unroll
        for (int j = 0; j < BT; ++j) v[j] = p + j < seg ? ld_dev(a0 + (size_t)(p + j) * SV + e) : 0.f;
#pragma unroll
        for (int j = 0; j < BT; ++j) acc += v[j];
      }
      sbuf[e] = failed ? __builtin_nanf("") : acc;
    }
  }
  __syncthreads();
  f32x4_t cS[NTW], cZ = zero4();
#pragma unroll
  for (int k = 0; k < NTW; ++k) {
    const int mb = (w + 4 * k) / DB;
#pragma unroll
    for (int r = 0; r < 4; ++r) cS[k][r] = sbuf[(16 * db + 4 * g + r) * M + 16 * mb + r16];
  }
  if (zw) {
#pragma unroll
    for (int r = 0; r < 4; ++r) cZ[r] = sbuf[D * M + 16 * db + 4 * g + r];
  }
  auto write_state = [&](const f32x4_t* s_, const f32x4_t& z_, float* dS, float* dZ) {
    store_S_tiles<D, M, NTW>(dS, s_, w, r16, g);
    if (zw && r16 == 0) *reinterpret_cast<float4*>(dZ + 16 * db + 4 * g) = make_float4(z_[0], z_[1], z_[2], z_[3]);
  };
  if (ckpt) {
    float* ck = ckpt + ((size_t)bh * (nseg + 1) + seg) * SV;
    write_state(cS, cZ, ck, ck + D * M);
  }
  if (seg == nseg - 1 && (ckpt || S_out)) {
    f32x4_t fS[NTW], fZ = cZ + accZ;
#pragma unroll
    for (int k = 0; k < NTW; ++k) fS[k] = cS[k] + accS[k];
    if (ckpt) {
      float* ck = ckpt + ((size_t)bh * (nseg + 1) + nseg) * SV;
      write_state(fS, fZ, ck, ck + D * M);
    }
    if (S_out) write_state(fS, fZ, S_out + (size_t)bh * D * M, Z_out + (size_t)bh * D);
  }
  stage(cS, cZ);
  __syncthreads();

  // O = (num + S_c^T phi(Q)) / (den + phi(Q).Z_c)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int c0 = t0 + c * CH;
    if (c0 < t1) {
      const int il = 16 * w + r16;
      const bool row_ok = il < t1 - c0;
      f32x4_t dn = zero4();
#pragma unroll
      for (int s = 0; s < DS; ++s) mmaf<P::FZ, P::FQ>(dn, zr.template frag<P::FZ>(r16, 32 * s, g), qk[c][s]);
      const float den = dl[c] + dn[0];
      const float inv = 1.f / den;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4_t acc = num[c][mb];
#pragma unroll
        for (int s = 0; s < DS; ++s)
          mmaf<P::FS, P::FQ>(acc, st.template frag<P::FS>(16 * mb + r16, 32 * s, g), qk[c][s]);
        if (row_ok) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = acc[r] * inv;
          IO<T>::store4(Oh + (size_t)(c0 + il) * M + 16 * mb + 4 * g, o);
        }
      }
      if (den_out && g == 0 && row_ok) den_out[(size_t)bh * N + c0 + il] = den;
    }
  }
}

// Clears the one-pass forward's `sync` words (n of them) before its launch.
__global__ __launch_bounds__(NT) void k_sync_clear(unsigned* __restrict__ sync, int n) {
  for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT) sync[i] = 0u;
}

// Prefix states from segment aggregates: pref[bh][s] = init + sum_{t<s}
// agg[bh][t], s = 0..nseg (init = (S0, Z0) or zero), summed in segment
// order; with last_only, only the total (entry nseg) is written.  One thread
// per state element; the aggregates are read in batches so that many loads
// are in flight.
template <int D, int M>
__global__ __launch_bounds__(NT) void k_scan_states(const float* __restrict__ agg, const float* __restrict__ S0,
                                                     const float* __restrict__ Z0, float* __restrict__ pref,
                                                     int nseg, int last_only) {
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
  float* o = pref + (size_t)bh * (nseg + 1) * SV + e;
  for (int s0 = 0; s0 < nseg; s0 += BT) {
    float v[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) v[j] = s0 + j < nseg ? a[(size_t)(s0 + j) * SV] : 0.f;
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      if (s0 + j < nseg) {
        if (!last_only) o[(size_t)(s0 + j) * SV] = run;
        run += v[j];
      }
    }
  }
  o[(size_t)nseg * SV] = run;
}

// Suffix states of the reverse aggregates, in place: ragg[bh][s] <- sum over
// p > s of ragg[bh][p], summed from the last segment down.
template <int D, int M>
__global__ __launch_bounds__(NT) void k_scan_rev(float* __restrict__ ragg, int nseg) {
  constexpr int SV = D * M + D, BT = 16;
  const int bh = blockIdx.x;
  const int e = blockIdx.y * NT + threadIdx.x;
  if (e >= SV) return;
  float* a = ragg + (size_t)bh * nseg * SV + e;
  float run = 0.f;
  for (int s1 = nseg; s1 > 0; s1 -= BT) {
    const int s0 = s1 - BT;
    float v[BT];
#pragma unroll
    for (int j = 0; j < BT; ++j) v[j] = s0 + j >= 0 ? a[(size_t)(s0 + j) * SV] : 0.f;
#pragma unroll
    for (int j = BT - 1; j >= 0; --j) {
      if (s0 + j >= 0) {
        a[(size_t)(s0 + j) * SV] = run;
        run += v[j];
      }
    }
  }
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

// ============================================================ non-causal B
// Non-causal backward (reading notes on "Transformers are RNNs", section 3.2,
// eq. 5-6; the causal backward's quotient rule with the masks removed): with
// the totals S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j) and, per query,
// u_i = S dO_i, den_i = phi(Q_i).Z, O_i.dO_i = phi(Q_i).u_i / den_i,
//   dphiQ_i = (u_i - Z (O_i.dO_i)) / den_i,
//   R = sum_i phi(Q_i) g_i^T, r = sum_i c_i phi(Q_i)  (g_i = dO_i / den_i,
//     c_i = -(O_i.dO_i) / den_i),
//   dphiK_j = R V_j + r,  dV_j = R^T phi(K_j).
// Totals come from S_t/Z_t when given (the forward's), else from entry nseg
// of a scanned prefix array `pref`, else from summing all segment aggregates
// `agg` here.

// Stage a state total (S then Z, row-major [d][m]) into planes and a float32 vector.
template <int D, int M, int NP, int NTH>
__device__ __forceinline__ void stage_total(Planes<NP, D, M>& sp, float* sz, float* sbuf, const float* pref,
                                            const float* agg, int nseg, const float* St = nullptr,
                                            const float* Zt = nullptr) {
  constexpr int SV = D * M + D;
  const float* src;
  if (St) {  // the totals as given ([D][M] and [D])
    for (int e = 4 * threadIdx.x; e < SV; e += 4 * NTH) {
      if (e < D * M) {
        const float4 a = *reinterpret_cast<const float4*>(St + e);
        const float x[4] = {a.x, a.y, a.z, a.w};
        sp.put4(e / M, e % M, x);
      } else {
        *reinterpret_cast<float4*>(sz + (e - D * M)) = *reinterpret_cast<const float4*>(Zt + (e - D * M));
      }
    }
    return;
  }
  if (pref) {
    src = pref + (size_t)nseg * SV;
  } else {
    sum_states<D, M, NTH>(sbuf, nullptr, nullptr, agg, 0, nseg);
    __syncthreads();
    src = sbuf;
  }
  for (int e = 4 * threadIdx.x; e < SV; e += 4 * NTH) {
    const float4 a = *reinterpret_cast<const float4*>(src + e);
    if (e < D * M) {
      const float x[4] = {a.x, a.y, a.z, a.w};
      sp.put4(e / M, e % M, x);
    } else {
      *reinterpret_cast<float4*>(sz + (e - D * M)) = a;
    }
  }
}

// Query pass: dQ, and the reverse aggregates (R^T, r) of each segment.
// Feature slices (ns per value head, la_wide.h) see only their shares of den_i
// = phi(Q_i) . Z and of num_i . dO_i = phi(Q_i)^T S dO_i: as in the causal
// query pass (la_bwd2.h), MODE kNcShares writes the slice's two shares of
// token i to gc[bh][i] and nothing else, and kNcGiven reads the pair (1/den_i,
// O_i . dO_i) of value head bh / ns, formed from their sums, from gc.
constexpr int kNcFull = 0, kNcGiven = 1, kNcShares = 2;
template <typename T, int D, int M, int MODE = kNcFull>
__global__ __launch_bounds__(NT) void k_nc_qr(const T* __restrict__ Q, const T* __restrict__ dO,
                                               const float* __restrict__ St, const float* __restrict__ Zt,
                                               const float* __restrict__ agg, const float* __restrict__ pref,
                                               T* __restrict__ dQ, float* __restrict__ ragg, int N, int L, int nseg, int fm,
                                               int ns, float2* __restrict__ gc) {
  using P = Prec<T>;
  constexpr int DB = D / 16, NTW = DB * (M / 16) / 4, SV = D * M + D;
  constexpr int E = IO<T>::E;
  __shared__ Planes<cmax(P::NQ, P::dR), CH, D> qt;  // phi(Q)
  __shared__ Planes<P::NDO, CH, M> ot;               // dO
  __shared__ Planes<P::NG, CH, M + 16> gt;           // [g | c | 0]
  __shared__ Planes<P::NS, D, M> sp;                 // S total, [d][m]
  __shared__ alignas(16) float sZ[D];                // Z total

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const int db = w % DB;
  const bool zw = w < DB;
  const int vh = MODE != kNcFull ? bh / ns : bh;  // value head
  const T* Qh = Q + (size_t)bh * N * D;
  const T* dOh = dO + (size_t)vh * N * M;
  static_assert(sizeof(gt.v) >= SV * sizeof(float), "g planes too small to hold a float32 state");
  stage_total<D, M, P::NS, NT>(sp, sZ, reinterpret_cast<float*>(&gt.v[0][0][0]),
                               pref ? pref + (size_t)bh * (nseg + 1) * SV : nullptr,
                               agg ? agg + (size_t)bh * nseg * SV : nullptr, nseg,
                               St ? St + (size_t)bh * D * M : nullptr, Zt ? Zt + (size_t)bh * D : nullptr);
  __syncthreads();
  gt.zero_cols(M + 1, M + 16);

  f32x4_t acc[NTW], accr = zero4();  // R^T layout; accr[0] on lanes g = 0 is r[16db + r16]
#pragma unroll
  for (int k = 0; k < NTW; ++k) acc[k] = zero4();

  RowBuf<T, CH, D> bq[2];
  RowBuf<T, CH, M> bd[2];
  auto fetch = [&](RowBuf<T, CH, D>& q_, RowBuf<T, CH, M>& d_, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      q_.load(Qh + (size_t)c0 * D, nv);
      d_.load(dOh + (size_t)c0 * M, nv);
    }
  };
  auto chunk = [&](RowBuf<T, CH, D>& q_, RowBuf<T, CH, M>& d_, int c0) {
    const int nv = min(CH, t1 - c0);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    q_.template stage_phi<cmax(P::NQ, P::dR), CH, D, 8>(qt, nv, nullptr, fm);
    d_.stage_values(ot);
    fetch(q_, d_, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    {
      const int il = 16 * w + r16;
      const bool row_ok = il < nv;
      Frag<P::U1_b> dof[M / 32];
#pragma unroll
      for (int s = 0; s < M / 32; ++s) dof[s] = ot.template frag<P::U1_b>(il, 32 * s, g);
      f32x4_t U[DB];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        f32x4_t u = zero4();
#pragma unroll
        for (int s = 0; s < M / 32; ++s)
          mmaf<P::U1_a, P::U1_b>(u, sp.template frag<P::U1_a>(16 * d0 + r16, 32 * s, g), dof[s]);
        U[d0] = u;  // S dO_i   [d][i]
      }
      float pu = 0.f, pz = 0.f, qv[DB][4], zv[DB][4];
#pragma unroll
      for (int d0 = 0; d0 < DB; ++d0) {
        // phi(Q) as the sum of its planes (float32 level with three, 2^-16
        // relative with two); den and O.dO below are formed from these same
        // values, so the cancellation in dphiQ stays exact
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
      if constexpr (MODE == kNcShares) {
        if (g == 0 && row_ok) gc[(size_t)bh * N + c0 + il] = make_float2(pu, pz);
        return;  // the shares are all this mode writes
      }
      float invz = row_ok ? 1.f / pz : 0.f;
      float odo = row_ok ? pu * invz : 0.f;  // O_i . dO_i
      if constexpr (MODE == kNcGiven) {
        const float2 pr = row_ok ? gc[(size_t)vh * N + c0 + il] : make_float2(0.f, 0.f);
        invz = pr.x;
        odo = pr.y;
      }
      if (row_ok) {
#pragma unroll
        for (int d0 = 0; d0 < DB; ++d0) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (U[d0][r] - zv[d0][r] * odo) * invz * dfeat(qv[d0][r], fm);
          IO<T>::store4(dQ + (size_t)bh * N * D + (size_t)(c0 + il) * D + 16 * d0 + 4 * g, o);
        }
      }
#pragma unroll
      for (int mm = 0; mm < M / 4; mm += 4) {
        float dv[4];
        ot.get4(il, g * (M / 4) + mm, dv);
#pragma unroll
        for (int q = 0; q < 4; ++q) dv[q] *= invz;
        gt.put4(il, g * (M / 4) + mm, dv);
      }
      if (g == 0) gt.put1(il, M, -odo * invz);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
      const Frag<P::dR> qb = qt.template tfrag<P::dR>(32 * s, 16 * db, g, r16);
#pragma unroll
      for (int k = 0; k < NTW; ++k) {
        const int mb = (w + 4 * k) / DB;
        mmaf<P::dR, P::dR>(acc[k], gt.template tfrag<P::dR>(32 * s, 16 * mb, g, r16), qb);
      }
      if (zw) mmaf<P::dR, P::dR>(accr, gt.template tfrag<P::dR>(32 * s, M, g, r16), qb);
    }
  };
  fetch(bq[0], bd[0], t0);
  fetch(bq[1], bd[1], t0 + CH);
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(bq[0], bd[0], c0);
    if (c0 + CH < t1) chunk(bq[1], bd[1], c0 + CH);
  }
  if constexpr (MODE != kNcShares) {
    float* out = ragg + ((size_t)bh * nseg + seg) * SV;
    store_ST_tiles<D, M, NTW>(out, acc, w, r16, g);
    if (zw && g == 0) out[D * M + 16 * db + r16] = accr[0];
  }
}

// Key pass: dK = (R V_j + r) phi'(K_j), dV = R^T phi(K_j) with the totals R, r.
// PART (feature slices, ns per value head, la_wide.h): dV sums over all of a
// head's features, so each slice writes its share (float32, [bh][n][M] in
// pdv), summed over the slices afterwards.
template <typename T, int D, int M, bool PART = false>
__global__ __launch_bounds__(NT) void k_nc_kv(const T* __restrict__ K, const T* __restrict__ V,
                                               const float* __restrict__ ragg, const float* __restrict__ rpref,
                                               T* __restrict__ dK, T* __restrict__ dV, int N, int L, int nseg, int fm,
                                               int ns, float* __restrict__ pdv) {
  using P = Prec<T>;
  constexpr int DB = D / 16, MB = M / 16, SV = D * M + D;
  constexpr int NKT = P::VR, NVT = cmax(P::KR_b, 1);
  __shared__ Planes<cmax(NKT, 1), CH, D> kt;  // phi(K)
  __shared__ Planes<cmax(P::NV, NVT), CH, M> vt;
  __shared__ Planes<P::NR, D, M> rp;          // R total, [d][m]
  __shared__ alignas(16) float k32[CH][D + 4];
  __shared__ alignas(16) float sr[D];         // r total

  const int item = seg_item(nseg), seg = item % nseg, bh = item / nseg;
  const int t0 = seg * L, t1 = min(N, t0 + L);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g = l >> 4;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)(PART ? bh / ns : bh) * N * M;
  static_assert(sizeof(kt.v) >= SV * sizeof(float), "key planes too small to hold a float32 state");
  stage_total<D, M, P::NR, NT>(rp, sr, reinterpret_cast<float*>(&kt.v[0][0][0]),
                               rpref ? rpref + (size_t)bh * (nseg + 1) * SV : nullptr,
                               ragg + (size_t)bh * nseg * SV, nseg);

  RowBuf<T, CH, D> bk[2];
  RowBuf<T, CH, M> bv[2];
  auto fetch = [&](RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    if (nv > 0) {
      k_.load(Kh + (size_t)c0 * D, nv);
      v_.load(Vh + (size_t)c0 * M, nv);
    }
  };
  auto chunk = [&](RowBuf<T, CH, D>& k_, RowBuf<T, CH, M>& v_, int c0) {
    const int nv = min(CH, t1 - c0);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    k_.template stage_phi<cmax(NKT, 1), CH, D, 8, D + 4>(kt, nv, &k32[0][0], fm);
    v_.stage_values(vt);
    fetch(k_, v_, c0 + 2 * CH);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    const int jl = 16 * w + r16;
    const bool row_ok = jl < nv;
    Frag<NVT> vfr[M / 32];
#pragma unroll
    for (int s = 0; s < M / 32; ++s) vfr[s] = vt.template frag<NVT>(jl, 32 * s, g);
#pragma unroll
    for (int d0 = 0; d0 < DB; ++d0) {
      f32x4_t a = zero4();
#pragma unroll
      for (int s = 0; s < M / 32; ++s)
        mmaf<P::KR_a, P::KR_b>(a, rp.template frag<P::KR_a>(16 * d0 + r16, 32 * s, g), vfr[s]);
      if (row_ok) {
        const float4 k4 = *reinterpret_cast<const float4*>(&k32[jl][16 * d0 + 4 * g]);
        const float4 r4 = *reinterpret_cast<const float4*>(&sr[16 * d0 + 4 * g]);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w}, rr[4] = {r4.x, r4.y, r4.z, r4.w};
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (a[r] + rr[r]) * dfeat(kv[r], fm);
        IO<T>::store4(dK + (size_t)bh * N * D + (size_t)(c0 + jl) * D + 16 * d0 + 4 * g, o);
      }
    }
    Frag<NKT> kfr[D / 32];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kfr[s] = kt.template frag<NKT>(jl, 32 * s, g);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t a = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        mmaf<P::VR, P::VR>(a, rp.template tfrag<P::VR>(32 * s, 16 * mb, g, r16), kfr[s]);
      if (row_ok) {
        if constexpr (PART) {
          *reinterpret_cast<float4*>(pdv + ((size_t)bh * N + c0 + jl) * M + 16 * mb + 4 * g) =
              make_float4(a[0], a[1], a[2], a[3]);
        } else {
          float o[4] = {a[0], a[1], a[2], a[3]};
          IO<T>::store4(dV + (size_t)bh * N * M + (size_t)(c0 + jl) * M + 16 * mb + 4 * g, o);
        }
      }
    }
  };
  fetch(bk[0], bv[0], t0);
  fetch(bk[1], bv[1], t0 + CH);
  for (int c0 = t0; c0 < t1; c0 += 2 * CH) {
    chunk(bk[0], bv[0], c0);
    if (c0 + CH < t1) chunk(bk[1], bv[1], c0 + CH);
  }
}

// ================================================================= decode
// One RNN step per head (eq. 18-20): S += phi(k) v^T, Z += phi(k),
// y = phi(q)^T S / phi(q)^T Z; with a log-decay per head ("Linear
// Attention/zh", RetNet and gated variants) S = a S + phi(k) v^T and
// Z = a Z + phi(k), a = exp(logA[head]).  One wavefront per head streams the head's
// D x M float32 state through registers in 1 KiB coalesced rows per
// instruction, updates it in place and reduces phi(q)^T S across lanes.
template <typename T, int D, int M>
__global__ __launch_bounds__(NT) void k_decode(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, const float* __restrict__ logA,
                                                float* __restrict__ S, float* __restrict__ Z, T* __restrict__ y,
                                                int BH, int fm) {
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
  const float a = live && logA ? __builtin_amdgcn_exp2f(logA[head] * 1.4426950408889634f) : 1.f;
  if (live) {
    if (l < D) {
      sq[w][l] = feat(ld(q + (size_t)head * D + l), fm);
      const float pk = feat(ld(k + (size_t)head * D + l), fm);
      sk[w][l] = pk;
      zn = a * Z[(size_t)head * D + l] + pk;
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
    s.x = a * s.x + pk * v0;
    s.y = a * s.y + pk * v1;
    s.z = a * s.z + pk * v2;
    s.w = a * s.w + pk * v3;
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
