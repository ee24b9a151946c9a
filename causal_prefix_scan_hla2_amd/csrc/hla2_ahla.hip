// hla2_ahla.hip -- AHLA, the asymmetric variant of the technical summary of
// arXiv 2510.27258 on gist.science (§2): the operator Q (K^T Q)(K^T V), causally
// masked, row t
//     num_t = sum_{j<=t} sum_{i<=j} g^(t-i) (q_t.k_j)(q_j.k_i) v_i,   den_t likewise with v_i -> 1,
// i.e. A_g A_g V with A_g = L o D o (Q K^T).  Streaming summaries (the page
// names them P^KV, m^K, E, n): P' = [P^KV | m^K] = sum g^(t-i) k_i v'_i^T with
// v' = [v | 1], and E' = [E | n] = sum_j g^(t-j) k_j y_j^T with y_j = P'_j^T q_j;
// then [num | den]_t = E'_t^T q_t.
//
// Chunk-parallel form (chunks of BC tokens, local index tau, Ad = L o D1 o (Q K^T)):
//     Y = diag(g^(tau+1)) Q P0' + Ad V',     O = diag(g^(tau+1)) Q E0' + Ad Y,
//     P' <- g^BC P' + K^T diag(g^(BC-1-i)) V',   E' <- g^BC E' + K^T diag(g^(BC-1-j)) Y,
// and two consecutive segments A, B combine as
//     P' = G_B P'_A + P'_B,   E' = G_B E'_A + E'_B + G_B M_B P'_A,   M = M_A + M_B,
// with M_B = sum_{j in B} k_j q_j^T (no decay: the powers of j cancel).
// Three launches, as for the second-order forward: segment summaries, the
// exclusive scan over segments, and the output walk from each segment's prefix.
#include "hla2_internal.h"
#include "hla2_tiles.h"

namespace hla2 {

// Under the ratio with bf16 operands the carried state (P', E') and Y enter their products as two
// bf16 halves (hla2_tiles.h): the ratio of two AHLA sums cancels, and with one bf16 rounding of each
// operand the rel-L2 of o over the well-conditioned tokens of 32 heads of 2048 tokens (d = dv = 64)
// is 2.0e-2 measured; with these three split a CPU model of the chunk walk's rounding points gives
// 0.7e-2 (splitting Ad as well buys little more).
template <typename T, bool NORM>
constexpr bool ahla_split() { return NORM && sizeof(T) == 2; }

template <typename T, int DK, int DVP, int BC, bool SPLIT>
struct AhlaCfg {
  static constexpr int PAD = lds_pad_bytes<T>() / sizeof(T);
  static constexpr int LDQ = DK + PAD, LDV = DVP + PAD, LDC = BC + PAD;
  // With SPLIT, E' is copied into P''s slot once Y is formed (P' is read only for Y), so that the low
  // halves of Y and of the state copy fit beside it.
  static constexpr int Q_OFF = 0, K_OFF = BC * LDQ, V_OFF = K_OFF + BC * LDQ, Y_OFF = V_OFF + BC * LDV,
                       AD_OFF = Y_OFF + BC * LDV, P_OFF = AD_OFF + BC * LDC,
                       E_OFF = SPLIT ? P_OFF : P_OFF + DK * LDV, YL_OFF = E_OFF + DK * LDV,
                       PL_OFF = YL_OFF + BC * LDV, EL_OFF = PL_OFF,
                       ELEMS = SPLIT ? PL_OFF + DK * LDV : E_OFF + DK * LDV;
};

// LDS bytes of one walker workgroup: the element rows, then the decay table and den.
template <typename T, int DK, int DVP, int BC, bool SPLIT>
constexpr int ahla_lds_bytes() {
  return AhlaCfg<T, DK, DVP, BC, SPLIT>::ELEMS * (int)sizeof(T) + (2 * BC + 3) * 4 + BC * 4;
}

// Summary mode (OUT = false): a segment from the zero state, writing P' | E' | M.  Output
// mode: a segment from its scanned prefix P' | E'.  With LEAD (output mode, segment 0) the
// state after the segment is written as the prefix of segment 1.
template <typename T, int DK, int DV, int DVP, int BC, bool OUT, bool NORM, bool LEAD>
__device__ __forceinline__ void ahla_walk_body(const AhlaArgs &a, const int bh, const int seg, unsigned char *lds) {
  constexpr bool SPLIT = ahla_split<T, NORM>();
  using Cfg = AhlaCfg<T, DK, DVP, BC, SPLIT>;
  static_assert((Cfg::ELEMS * sizeof(T)) % 4 == 0, "decay table alignment");
  T *const smem = (T *)lds;
  float *const pw = (float *)(lds + Cfg::ELEMS * sizeof(T));
  float *const dens = pw + (2 * BC + 3);
  T *const Qs = smem + Cfg::Q_OFF, *const Ks = smem + Cfg::K_OFF, *const Vs = smem + Cfg::V_OFF;
  T *const Ys = smem + Cfg::Y_OFF, *const Ads = smem + Cfg::AD_OFF, *const Ps = smem + Cfg::P_OFF;
  T *const Es = smem + Cfg::E_OFF, *const Yls = smem + Cfg::YL_OFF, *const Pls = smem + Cfg::PL_OFF;
  T *const Els = smem + Cfg::EL_OFF;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, nn = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = ahla_seg_chunk0(a, seg) * a.kc, tokE = min(a.n, tok0 + ahla_seg_chunks(a, seg) * a.kc);
  const int nch = (tokE - tok0 + BC - 1) / BC;
  const long hq = (long)bh * a.n * a.d, hv = (long)bh * a.n * a.dv;
  const T *qh = (const T *)a.q + hq, *kh = (const T *)a.k + hq, *vh = (const T *)a.v + hv;
  for (int e = tid; e < 2 * BC + 3; e += BWD_THREADS) pw[e] = exp2f((float)e * a.log2g);
  constexpr long PB = 2L * DK * DVP, SB = 2L * DK * DVP + (long)DK * DK;

  using TU = TileCount<DK, DVP>;
  f32x4 P[TU::PER], E[TU::PER];
  // with a prologue fold (below) segment 2 starts from segment 1's prefix
  const bool pfold = OUT && !LEAD && a.pfold && seg == 2;
  const float *pref = (OUT && seg > 0) ? a.prefix + ((long)bh * a.nseg + (pfold ? 1 : seg)) * PB : nullptr;
  for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
    const int o = (i0 + nn) * DVP + j0 + 4 * gq;
    P[it] = pref ? *(const f32x4 *)(pref + o) : zero4();
    E[it] = pref ? *(const f32x4 *)(pref + DK * DVP + o) : zero4();
  });
  using TM = TileCount<DK, DK>;
  f32x4 M[OUT ? 1 : TM::PER];
#pragma unroll
  for (int i = 0; i < (OUT ? 1 : TM::PER); ++i) M[i] = zero4();

  RowTile<T, BC, DK> rq, rk;
  RowTile<T, BC, DVP> rv;
  rq.fetch(qh, a.d, tok0, a.n, -1, tid);
  rk.fetch(kh, a.d, tok0, a.n, -1, tid);
  rv.fetch(vh, a.dv, tok0, a.n, NORM ? DV : -1, tid);

  // Prologue fold (a three-segment lead plan has no scan launch): segment 2 folds segment 1's
  // summary (P'_1, E'_1, M_1) onto segment 1's prefix with the scan's combine,
  //   E' <- G E' + E'_1 + G M_1 P',   P' <- G P' + P'_1   (G = decay^(tokens per segment)),
  // the product on MFMA from M_1 and P' in LDS (two-term operands under the ratio), while the
  // first chunk's rows are in flight.  The Q, K and P' slots are free until the walk starts; M_1's
  // halves take the Q and K slots, which hold DK rows when the chunk is DK tokens (d = 64).
  if constexpr (OUT && !LEAD && BC == DK) {
    if (pfold) {
      const float G = a.gseg;
      const float *sb = a.sums + ((long)bh * (a.nseg - 1) + 1) * SB, *Ms = sb + 2 * DK * DVP;
      for (int e = 4 * tid; e < DK * DK; e += 4 * BWD_THREADS)
        st4_split<SPLIT>(Qs, Ks, Cfg::LDQ, e / DK, e % DK, *(const f32x4 *)(Ms + e));
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        if (ok) st4_split<SPLIT>(Ps, Pls, Cfg::LDV, i0 + nn, j0 + 4 * gq, P[it]);
      });
      __syncthreads();
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
        f32x4 x = pt2x<SPLIT, false, false, DK>(zero4(), Qs, Ks, Cfg::LDQ, Ps, Cfg::LDV, i0, j0, lane);
        if constexpr (SPLIT) x = pt<false, false, DK>(x, Qs, Cfg::LDQ, Pls, Cfg::LDV, i0, j0, lane);
        const int o = (i0 + nn) * DVP + j0 + 4 * gq;
        E[it] = G * E[it] + *(const f32x4 *)(sb + DK * DVP + o) + G * x;
        P[it] = G * P[it] + *(const f32x4 *)(sb + o);
      });
      __syncthreads();  // every read of the staged operands done
    }
  }

  for (int ch = 0; ch < nch; ++ch) {
    const int t0 = tok0 + ch * BC;
    // state copies for this chunk's products, and its rows
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) {
        st4_split<SPLIT>(Ps, Pls, Cfg::LDV, i0 + nn, j0 + 4 * gq, P[it]);
        if (OUT && !SPLIT) st4l(Es, Cfg::LDV, i0 + nn, j0 + 4 * gq, E[it]);
      }
    });
    rq.put(Qs, Cfg::LDQ, tid);
    rk.put(Ks, Cfg::LDQ, tid);
    rv.put(Vs, Cfg::LDV, tid);
    __syncthreads();
    {
      const int tn = tok0 + min(ch + 1, nch - 1) * BC;
      rq.fetch(qh, a.d, tn, a.n, -1, tid);
      rk.fetch(kh, a.d, tn, a.n, -1, tid);
      rv.fetch(vh, a.dv, tn, a.n, NORM ? DV : -1, tid);
    }
    // Ad = L o D1 o (Q K^T)
    for_tiles<BC, BC>(w, [&](int i0, int j0, bool ok, int) {
      f32x4 x = pt<false, true, DK>(zero4(), Qs, Cfg::LDQ, Ks, Cfg::LDQ, i0, j0, lane);
      const int tr = i0 + nn;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ti = j0 + 4 * gq + e;
        // the factor is read and applied on every lane (clamped index, masked value) so
        // that no branch forms around the table read
        x[e] = (ti <= tr ? x[e] : 0.f) * pw[ti <= tr ? tr - ti : 0];
      }
      if (ok) st4l(Ads, Cfg::LDC, tr, j0 + 4 * gq, x);
    });
    __syncthreads();
    // Y = diag(g^(tau+1)) Q P0' + Ad V'
    for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int) {
      f32x4 x = pt2y<SPLIT, false, false, DK>(zero4(), Qs, Cfg::LDQ, Ps, Pls, Cfg::LDV, i0, j0, lane);
      x *= pw[i0 + nn + 1];
      x = pt<false, false, BC>(x, Ads, Cfg::LDC, Vs, Cfg::LDV, i0, j0, lane);
      if (ok) st4_split<SPLIT>(Ys, Yls, Cfg::LDV, i0 + nn, j0 + 4 * gq, x);
    });
    __syncthreads();
    if constexpr (OUT && SPLIT) {  // every read of P''s copy is done: E' takes its slot
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        if (ok) st4_split<SPLIT>(Es, Els, Cfg::LDV, i0 + nn, j0 + 4 * gq, E[it]);
      });
      __syncthreads();
    }
    // outputs O = diag(g^(tau+1)) Q E0' + Ad Y (kept in registers until den is known)
    f32x4 O[OUT ? TileCount<BC, DVP>::PER : 1];
    if constexpr (OUT) {
      for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        f32x4 x = pt2y<SPLIT, false, false, DK>(zero4(), Qs, Cfg::LDQ, Es, Els, Cfg::LDV, i0, j0, lane);
        x *= pw[i0 + nn + 1];
        x = pt2y<SPLIT, false, false, BC>(x, Ads, Cfg::LDC, Ys, Yls, Cfg::LDV, i0, j0, lane);
        O[it] = x;
        if (NORM && ok && j0 + 4 * gq == DV) dens[i0 + nn] = x[0];
      });
    } else {
      // M += K^T Q (no decay)
      for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
        M[it] = pt<true, false, BC>(M[it], Ks, Cfg::LDQ, Qs, Cfg::LDQ, i0, j0, lane);
      });
    }
    // P' <- g^BC P' + K^T diag(g^(BC-1-i)) V';  E' <- g^BC E' + K^T diag(g^(BC-1-j)) Y
    const float gB = pw[BC];
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
      P[it] = ptw<true, false, BC>(gB * P[it], Ks, Cfg::LDQ, Vs, Cfg::LDV, i0, j0, lane,
                                   [&](int i) { return pw[BC - 1 - i]; });
      E[it] = ptw<true, false, BC>(gB * E[it], Ks, Cfg::LDQ, Ys, Cfg::LDV, i0, j0, lane,
                                   [&](int i) { return pw[BC - 1 - i]; });
      if constexpr (SPLIT)
        E[it] = ptw<true, false, BC>(E[it], Ks, Cfg::LDQ, Yls, Cfg::LDV, i0, j0, lane,
                                     [&](int i) { return pw[BC - 1 - i]; });
    });
    __syncthreads();  // dens complete; every read of this chunk's LDS done
    if constexpr (OUT) {
      T *oh = (T *)a.out + hv;
      for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        const int tr = i0 + nn, t = t0 + tr;
        f32x4 x = O[it];
        if (NORM && a.normalize) x *= 1.f / dens[tr];
        if (ok) st_out(oh, a.dv, t, j0 + 4 * gq, a.n, x);
      });
      if (NORM && a.den_out && tid < BC && t0 + tid < a.n) a.den_out[(long)bh * a.n + t0 + tid] = dens[tid];
    }
  }
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * (a.nseg - 1) + seg) * SB;
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      const int o = (i0 + nn) * DVP + j0 + 4 * gq;
      if (ok) {
        *(f32x4 *)(sb + o) = P[it];
        *(f32x4 *)(sb + DK * DVP + o) = E[it];
      }
    });
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) *(f32x4 *)(sb + 2 * DK * DVP + (i0 + nn) * DK + j0 + 4 * gq) = M[it];
    });
  }
  if constexpr (OUT && LEAD) {
    // the state after segment 0 is the prefix of segment 1 (the layout the prefix is read in)
    float *pb = a.prefix + ((long)bh * a.nseg + seg + 1) * PB;
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      const int o = (i0 + nn) * DVP + j0 + 4 * gq;
      if (ok) {
        *(f32x4 *)(pb + o) = P[it];
        *(f32x4 *)(pb + DK * DVP + o) = E[it];
      }
    });
  }
}

// Walks segments (OUT ? seg_lo .. nseg-1 : 0 .. nseg-2) of every head, one workgroup each.
template <typename T, int DK, int DV, int DVP, int BC, bool OUT, bool NORM>
__global__ void __launch_bounds__(BWD_THREADS) ahla_walk_kernel(AhlaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[ahla_lds_bytes<T, DK, DVP, BC, ahla_split<T, NORM>()>()];
  const int lo = OUT ? a.seg_lo : 0, nr = (OUT ? a.nseg : a.nseg - 1) - lo;
  ahla_walk_body<T, DK, DV, DVP, BC, OUT, NORM, false>(a, blockIdx.x / nr, lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head for its outputs and
// leave the prefix of segment 1; the rest summarise segments 1 .. nseg-2 of every head.
template <typename T, int DK, int DV, int DVP, int BC, bool NORM>
__global__ void __launch_bounds__(BWD_THREADS) ahla_lead_kernel(AhlaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[ahla_lds_bytes<T, DK, DVP, BC, ahla_split<T, NORM>()>()];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    ahla_walk_body<T, DK, DV, DVP, BC, true, NORM, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = a.nseg - 2;
    ahla_walk_body<T, DK, DV, DVP, BC, false, NORM, false>(a, i / nr, 1 + i % nr, lds);
  }
}

// Exclusive scan over segments, per (b, h), fp32 on VALU:
//   prefix_0 = 0;  P'_{r+1} = G P'_r + P'(seg r),  E'_{r+1} = G E'_r + E'(seg r) + G M(seg r) P'_r.
// Workgroup (bh, sp) owns rows 16 sp .. 16 sp + 15 of E' and writes those rows of
// every prefix; each workgroup of a head keeps the whole P' sequence in LDS
// (elementwise), so the workgroups never wait on each other.
template <int DK, int DVP>
__global__ void __launch_bounds__(256) ahla_scan_kernel(AhlaArgs a, float gseg) {
  constexpr long PB = 2L * DK * DVP, SB = 2L * DK * DVP + (long)DK * DK;
  // a thread owns 4 consecutive columns of a row of E' (each float4 read of P' feeds 4 FMAs)
  constexpr int EQ = 16 * DVP / 4, NEQ = (EQ + 255) / 256;
  __shared__ __attribute__((aligned(16))) float Pl[DK * DVP], Ml[16 * DK];
  const int tid = threadIdx.x, bh = blockIdx.x, sp = blockIdx.y, r0 = 16 * sp;
  float *pre = a.prefix + (long)bh * a.nseg * PB;
  const int rs = a.first;  // 1: the prefix of segment 1 is given (written by segment 0's walk)
  const float *given = pre + (long)rs * PB;
  for (int e = 4 * tid; e < DK * DVP; e += 1024)
    *(f32x4 *)(Pl + e) = rs ? *(const f32x4 *)(given + e) : zero4();
  f32x4 E[NEQ];  // E'[r0 + f][c0 .. c0 + 3] for group q = tid + 256 i: f = q / (DVP/4), c0 = 4 (q % (DVP/4))
#pragma unroll
  for (int i = 0; i < NEQ; ++i) {
    const int q = tid + 256 * i;
    const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
    E[i] = (rs && (EQ % 256 == 0 || q < EQ)) ? *(const f32x4 *)(given + DK * DVP + (r0 + f) * DVP + c0) : zero4();
  }
  for (int r = rs; r < a.nseg; ++r) {
    float *pr = pre + (long)r * PB;
    __syncthreads();  // Pl holds P'_r
#pragma unroll
    for (int i = 0; i < NEQ; ++i) {
      const int q = tid + 256 * i;
      if ((r > rs || rs == 0) && (EQ % 256 == 0 || q < EQ)) {  // a given prefix is in place
        const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
        *(f32x4 *)(pr + (r0 + f) * DVP + c0) = *(const f32x4 *)(Pl + (r0 + f) * DVP + c0);
        *(f32x4 *)(pr + DK * DVP + (r0 + f) * DVP + c0) = E[i];
      }
    }
    if (r == a.nseg - 1) break;
    const float *sb = a.sums + ((long)bh * (a.nseg - 1) + r) * SB, *Mr = sb + 2 * DK * DVP;
    for (int e = tid; e < 16 * DK; e += 256) Ml[e] = Mr[r0 * DK + e];  // the group's rows of M
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NEQ; ++i) {
      const int q = tid + 256 * i;
      if (EQ % 256 == 0 || q < EQ) {
        const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
        f32x4 acc = zero4();
#pragma unroll 8
        for (int g2 = 0; g2 < DK; ++g2) acc += Ml[f * DK + g2] * *(const f32x4 *)(Pl + g2 * DVP + c0);
        E[i] = gseg * (E[i] + acc) + *(const f32x4 *)(sb + DK * DVP + (r0 + f) * DVP + c0);
      }
    }
    __syncthreads();  // every read of P'_r done
    for (int e = 4 * tid; e < DK * DVP; e += 1024)
      *(f32x4 *)(Pl + e) = gseg * *(const f32x4 *)(Pl + e) + *(const f32x4 *)(sb + e);
  }
}

template <typename T, int DK, int DV, bool NORM>
static hipError_t launch_ahla_t(int phase, int BH, const AhlaArgs &a, float gseg, hipStream_t s) {
  constexpr int DVP = lds_walk_dvp(sizeof(T) == 4, DV, NORM);
  constexpr int BC = lds_walk_chunk(sizeof(T) == 4, DK);
  switch (phase) {
    case AHLA_SUMMARY:
      hipLaunchKernelGGL((ahla_walk_kernel<T, DK, DV, DVP, BC, false, NORM>), dim3(BH * (a.nseg - 1)),
                         dim3(BWD_THREADS), 0, s, a);
      return hipGetLastError();
    case AHLA_SCAN:
      hipLaunchKernelGGL((ahla_scan_kernel<DK, DVP>), dim3(BH, DK / 16), dim3(256), 0, s, a, gseg);
      return hipGetLastError();
    case AHLA_OUTPUT:
      hipLaunchKernelGGL((ahla_walk_kernel<T, DK, DV, DVP, BC, true, NORM>), dim3(BH * (a.nseg - a.seg_lo)),
                         dim3(BWD_THREADS), 0, s, a);
      return hipGetLastError();
    case AHLA_LEAD:
      if (a.nseg < 2 || a.nbh != BH) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ahla_lead_kernel<T, DK, DV, DVP, BC, NORM>), dim3(BH * (a.nseg - 1)), dim3(BWD_THREADS),
                         0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK, int DV>
static hipError_t launch_ahla_n(bool norm, int phase, int BH, const AhlaArgs &a, float gseg, hipStream_t s) {
  return norm ? launch_ahla_t<T, DK, DV, true>(phase, BH, a, gseg, s)
              : launch_ahla_t<T, DK, DV, false>(phase, BH, a, gseg, s);
}


hipError_t launch_ahla(int dtype, int DK, int DV, bool norm, int phase, int BH, const AhlaArgs &a, float gseg,
                       hipStream_t s) {
  if (dtype == 0) {
    if (DK == 16 && DV == 16) return launch_ahla_n<float, 16, 16>(norm, phase, BH, a, gseg, s);
    if (DK == 64 && DV == 64) return launch_ahla_n<float, 64, 64>(norm, phase, BH, a, gseg, s);
    return hipErrorInvalidValue;
  }
  if (DK == 64 && DV == 64) return launch_ahla_n<bf16, 64, 64>(norm, phase, BH, a, gseg, s);
  // without den the walks at d <= 64, dv > 64 run on the register-resident walker; the scan
  // between them is the same
  if (DK == 64 && DV == 128 && !norm && phase != AHLA_SCAN) return launch_ahla8(phase, BH, a, s);
  if (DK == 64 && DV == 128) return launch_ahla_n<bf16, 64, 128>(norm, phase, BH, a, gseg, s);
  if (DK == 128 && DV == 64) return launch_ahla_n<bf16, 128, 64>(norm, phase, BH, a, gseg, s);
  if (DK == 128 && DV == 128) return launch_ahla_n<bf16, 128, 128>(norm, phase, BH, a, gseg, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
