// hla2_ho3.hip -- third-order HLA (technical summary of arXiv 2510.27258 on
// gist.science, §3): the interaction A A^T A with A = Q K^T, masked so that no
// index passes t, row t
//   num_t = sum_{l<=t} sum_{j<=l} sum_{i<=l} g^((t-j)+(t-l)+(t-i)) (q_t.k_j)(q_l.k_j)(q_l.k_i) v_i,
// den_t likewise with v_i -> 1: num = (L o D_{g^2} o (A_g A^T)) (A_g V).  The three
// prefix moments the page names (key moment S, the key-value prefix P and,
// through the segment maps, the query moment) carry it; the cross summaries
// are folded into one corrected accumulator W' (d x (dv+1)):
//   z_t = S_t q_t,  y'_t = P'_t^T q_t,  W'_t = g^3 W'_{t-1} + z_t y'_t^T,  [num|den]_t = W'_t^T q_t.
//
// Chunk form (BC tokens, local tau, Ad = L o D1 o (Q K^T), D3[t][l] = g^(3(t-l))):
//   Z = diag(g^(tau+1)) Q S0 + Ad K,   Y = diag(g^(tau+1)) Q P0' + Ad V',
//   O = diag(g^(3(tau+1))) Q W0' + (L o D3 o (Q Z^T)) Y,
//   S <- g^BC S + K^T diag(g^(BC-1-i)) K,  P' <- g^BC P' + K^T diag(g^(BC-1-i)) V',
//   W' <- g^(3BC) W' + Z^T diag(g^(3(BC-1-l))) Y.
// A segment of L tokens (u = 0..L-1) folds an incoming (S_A, P'_A, W'_A) as
//   W' = g^(3L) W'_A + W'_B + S_A Q2 P'_A + S_A X1 + X2 P'_A,  S = g^L S_A + S_B,  P' = g^L P'_A + P'_B,
// with the segment maps (the page's segment-level linear maps)
//   Q2 = sum_u g^(3L-1-u) q_u q_u^T,  X1 = sum_u g^(3L-2-2u) q_u y'_u^T,  X2 = sum_u g^(3L-2-2u) z_u q_u^T
// over the segment's own (zero-start) z, y'.
#include "hla2_internal.h"
#include "hla2_tiles.h"

namespace hla2 {

// Under the ratio with bf16 operands the carried state (S, P', W') and the chunk weights Ad and Wm
// enter their products as two bf16 halves, hi = bf16(x) and lo = bf16(x - hi), about 16 significant
// bits.  The ratio of two third-order sums cancels: with one bf16 rounding of each operand the rel-L2
// of o over the well-conditioned tokens of 32 heads of 2048 tokens (d = dv = 64) is 2.0e-2, with these
// five split 0.9e-2 (a CPU model of the chunk walk's rounding points, which reproduces the measured
// 2.0e-2 and, with four split, 1.0e-2).  Z and Y stay single: their low halves do not fit in LDS.
template <typename T, bool NORM>
constexpr bool ho3_split() { return NORM && sizeof(T) == 2; }

template <typename T, int DK, int DVP, int BC, bool SPLIT>
struct Ho3Cfg {
  static constexpr int PAD = lds_pad_bytes<T>() / sizeof(T);
  static constexpr int LDQ = DK + PAD, LDV = DVP + PAD, LDC = BC + PAD;
  // With SPLIT the second BC x BC slot holds Ad's low half; Wm and its low half (written once Ad is
  // consumed) take the two slots of Ad; the low halves of S, P', W' follow W'.
  static constexpr int Q_OFF = 0, K_OFF = BC * LDQ, V_OFF = K_OFF + BC * LDQ, Y_OFF = V_OFF + BC * LDV,
                       Z_OFF = Y_OFF + BC * LDV, AD_OFF = Z_OFF + BC * LDQ, ADL_OFF = AD_OFF + BC * LDC,
                       WM_OFF = SPLIT ? AD_OFF : ADL_OFF, WML_OFF = ADL_OFF, S_OFF = ADL_OFF + BC * LDC, P_OFF = S_OFF + DK * LDQ,
                       W_OFF = P_OFF + DK * LDV, SL_OFF = W_OFF + DK * LDV, PL_OFF = SL_OFF + DK * LDQ,
                       WL_OFF = PL_OFF + DK * LDV, ELEMS = SPLIT ? WL_OFF + DK * LDV : SL_OFF;
  static constexpr long PB = (long)DK * DK + 2L * DK * DVP;                 // S | P' | W'
  static constexpr long SB = PB + 2L * DK * DK + (long)DK * DVP;            // ... | Q2 | X1 | X2
};

// LDS bytes of one walker workgroup: the element rows, then the decay table and den.
template <typename T, int DK, int DVP, int BC, bool SPLIT>
constexpr int ho3_lds_bytes() {
  return Ho3Cfg<T, DK, DVP, BC, SPLIT>::ELEMS * (int)sizeof(T) + (3 * BC + 4) * 4 + BC * 4;
}

// Summary mode (OUT = false): a segment from the zero state, writing S | P' | W' and its
// maps.  Output mode: a segment from its scanned prefix.  With LEAD (output mode, segment 0)
// the state after the segment is written as the prefix of segment 1.
template <typename T, int DK, int DV, int DVP, int BC, bool OUT, bool NORM, bool LEAD>
__device__ __forceinline__ void ho3_walk_body(const Ho3Args &a, const int bh, const int seg, unsigned char *lds) {
  constexpr bool SPLIT = ho3_split<T, NORM>();
  using Cfg = Ho3Cfg<T, DK, DVP, BC, SPLIT>;
  static_assert((Cfg::ELEMS * sizeof(T)) % 4 == 0, "decay table alignment");
  T *const smem = (T *)lds;
  float *const pw = (float *)(lds + Cfg::ELEMS * sizeof(T));
  float *const dens = pw + (3 * BC + 4);
  T *const Qs = smem + Cfg::Q_OFF, *const Ks = smem + Cfg::K_OFF, *const Vs = smem + Cfg::V_OFF;
  T *const Ys = smem + Cfg::Y_OFF, *const Zs = smem + Cfg::Z_OFF, *const Ads = smem + Cfg::AD_OFF;
  T *const Wms = smem + Cfg::WM_OFF, *const Ss = smem + Cfg::S_OFF, *const Ps = smem + Cfg::P_OFF;
  T *const Ws = smem + Cfg::W_OFF, *const Adls = smem + Cfg::ADL_OFF, *const Sls = smem + Cfg::SL_OFF;
  T *const Pls = smem + Cfg::PL_OFF, *const Wls = smem + Cfg::WL_OFF, *const Wmls = smem + Cfg::WML_OFF;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, nn = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = ahla_seg_chunk0(a, seg) * a.kc, tokE = min(a.n, tok0 + ahla_seg_chunks(a, seg) * a.kc);
  // summarised segments are full, cps chunks (segment 0 of a lead plan is never summarised)
  const int seglen = a.cps * a.kc;
  const int nch = (tokE - tok0 + BC - 1) / BC;
  const long hq = (long)bh * a.n * a.d, hv = (long)bh * a.n * a.dv;
  const T *qh = (const T *)a.q + hq, *kh = (const T *)a.k + hq, *vh = (const T *)a.v + hv;
  for (int e = tid; e < 3 * BC + 4; e += BWD_THREADS) pw[e] = exp2f((float)e * a.log2g);

  using TS = TileCount<DK, DK>;
  using TU = TileCount<DK, DVP>;
  f32x4 S[TS::PER], P[TU::PER], W[TU::PER];
  // with a prologue fold (below) segment 2 starts from segment 1's prefix
  const bool pfold = OUT && !LEAD && a.pfold && seg == 2;
  const float *pref = (OUT && seg > 0) ? a.prefix + ((long)bh * a.nseg + (pfold ? 1 : seg)) * Cfg::PB : nullptr;
  for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
    S[it] = pref ? *(const f32x4 *)(pref + (i0 + nn) * DK + j0 + 4 * gq) : zero4();
  });
  for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
    const int o = (i0 + nn) * DVP + j0 + 4 * gq;
    P[it] = pref ? *(const f32x4 *)(pref + DK * DK + o) : zero4();
    W[it] = pref ? *(const f32x4 *)(pref + DK * DK + DK * DVP + o) : zero4();
  });
  // segment maps (summary mode)
  f32x4 Q2[OUT ? 1 : TS::PER], X1[OUT ? 1 : TU::PER], X2[OUT ? 1 : TS::PER];
#pragma unroll
  for (int i = 0; i < (OUT ? 1 : TS::PER); ++i) Q2[i] = X2[i] = zero4();
#pragma unroll
  for (int i = 0; i < (OUT ? 1 : TU::PER); ++i) X1[i] = zero4();

  RowTile<T, BC, DK> rq, rk;
  RowTile<T, BC, DVP> rv;
  rq.fetch(qh, a.d, tok0, a.n, -1, tid);
  rk.fetch(kh, a.d, tok0, a.n, -1, tid);
  rv.fetch(vh, a.dv, tok0, a.n, NORM ? DV : -1, tid);

  // Prologue fold (a three-segment lead plan has no scan launch): segment 2 folds segment 1's
  // summary onto segment 1's prefix (S_A, P'_A, W'_A) with the segment combine,
  //   T = S_A Q2 + X2,  W' <- G^3 W'_A + W'_1 + T P'_A + S_A X1,  S <- G S_A + S_1,  P' <- G P'_A + P'_1,
  // the products on MFMA from operands staged in the slots that are free until the walk starts (two
  // bf16 halves under the ratio), while the first chunk's rows are in flight.  The Q, K, Z and Ad slots
  // take DK rows when the chunk is DK tokens.
  if constexpr (OUT && !LEAD && BC == DK) {
    static_assert(Cfg::LDC == Cfg::LDQ, "T's halves share one pitch");
    if (pfold) {
      const float G = a.gseg, G3 = G * G * G;
      const float *sb = a.sums + ((long)bh * (a.nseg - 1) + 1) * Cfg::SB;
      const float *Q2g = sb + Cfg::PB, *X1g = Q2g + DK * DK, *X2g = X1g + DK * DVP;
      for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int it) {
        if (ok) st4_split<SPLIT>(Ss, Sls, Cfg::LDQ, i0 + nn, j0 + 4 * gq, S[it]);
      });
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        if (ok) st4_split<SPLIT>(Ps, Pls, Cfg::LDV, i0 + nn, j0 + 4 * gq, P[it]);
      });
      for (int e = 4 * tid; e < DK * DK; e += 4 * BWD_THREADS)
        st4_split<SPLIT>(Qs, Ks, Cfg::LDQ, e / DK, e % DK, *(const f32x4 *)(Q2g + e));
      for (int e = 4 * tid; e < DK * DVP; e += 4 * BWD_THREADS)
        st4_split<SPLIT>(Vs, Ys, Cfg::LDV, e / DVP, e % DVP, *(const f32x4 *)(X1g + e));
      __syncthreads();
      // T = S_A Q2 + X2
      for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int) {
        f32x4 x = pt2x<SPLIT, false, false, DK>(zero4(), Ss, Sls, Cfg::LDQ, Qs, Cfg::LDQ, i0, j0, lane);
        if constexpr (SPLIT) x = pt<false, false, DK>(x, Ss, Cfg::LDQ, Ks, Cfg::LDQ, i0, j0, lane);
        x += *(const f32x4 *)(X2g + (i0 + nn) * DK + j0 + 4 * gq);
        if (ok) st4_split<SPLIT>(Zs, Ads, Cfg::LDQ, i0 + nn, j0 + 4 * gq, x);
      });
      __syncthreads();
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
        f32x4 x = pt2x<SPLIT, false, false, DK>(zero4(), Zs, Ads, Cfg::LDQ, Ps, Cfg::LDV, i0, j0, lane);
        if constexpr (SPLIT) x = pt<false, false, DK>(x, Zs, Cfg::LDQ, Pls, Cfg::LDV, i0, j0, lane);
        x = pt2x<SPLIT, false, false, DK>(x, Ss, Sls, Cfg::LDQ, Vs, Cfg::LDV, i0, j0, lane);
        if constexpr (SPLIT) x = pt<false, false, DK>(x, Ss, Cfg::LDQ, Ys, Cfg::LDV, i0, j0, lane);
        const int o = (i0 + nn) * DVP + j0 + 4 * gq;
        W[it] = G3 * W[it] + *(const f32x4 *)(sb + DK * DK + DK * DVP + o) + x;
        P[it] = G * P[it] + *(const f32x4 *)(sb + DK * DK + o);
      });
      for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
        S[it] = G * S[it] + *(const f32x4 *)(sb + (i0 + nn) * DK + j0 + 4 * gq);
      });
      __syncthreads();  // every read of the staged operands done
    }
  }

  for (int ch = 0; ch < nch; ++ch) {
    const int t0 = tok0 + ch * BC;
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) st4_split<SPLIT>(Ss, Sls, Cfg::LDQ, i0 + nn, j0 + 4 * gq, S[it]);
    });
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) {
        st4_split<SPLIT>(Ps, Pls, Cfg::LDV, i0 + nn, j0 + 4 * gq, P[it]);
        if (OUT) st4_split<SPLIT>(Ws, Wls, Cfg::LDV, i0 + nn, j0 + 4 * gq, W[it]);
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
      if (ok) st4_split<SPLIT>(Ads, Adls, Cfg::LDC, tr, j0 + 4 * gq, x);
    });
    __syncthreads();
    // Z = diag(g^(tau+1)) Q S0 + Ad K;  Y = diag(g^(tau+1)) Q P0' + Ad V'
    for_tiles<BC, DK>(w, [&](int i0, int j0, bool ok, int) {
      f32x4 x = pt2y<SPLIT, false, true, DK>(zero4(), Qs, Cfg::LDQ, Ss, Sls, Cfg::LDQ, i0, j0, lane);
      x *= pw[i0 + nn + 1];
      x = pt2x<SPLIT, false, false, BC>(x, Ads, Adls, Cfg::LDC, Ks, Cfg::LDQ, i0, j0, lane);
      if (ok) st4l(Zs, Cfg::LDQ, i0 + nn, j0 + 4 * gq, x);
    });
    for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int) {
      f32x4 x = pt2y<SPLIT, false, false, DK>(zero4(), Qs, Cfg::LDQ, Ps, Pls, Cfg::LDV, i0, j0, lane);
      x *= pw[i0 + nn + 1];
      x = pt2x<SPLIT, false, false, BC>(x, Ads, Adls, Cfg::LDC, Vs, Cfg::LDV, i0, j0, lane);
      if (ok) st4l(Ys, Cfg::LDV, i0 + nn, j0 + 4 * gq, x);
    });
    __syncthreads();
    f32x4 O[OUT ? TileCount<BC, DVP>::PER : 1];
    if constexpr (OUT) {
      // Wm = L o D3 o (Q Z^T)
      for_tiles<BC, BC>(w, [&](int i0, int j0, bool ok, int) {
        f32x4 x = pt<false, true, DK>(zero4(), Qs, Cfg::LDQ, Zs, Cfg::LDQ, i0, j0, lane);
        const int tr = i0 + nn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int l = j0 + 4 * gq + e;
          // the factor is read and applied on every lane (clamped index, masked value) so
          // that no branch forms around the table read
          x[e] = (l <= tr ? x[e] : 0.f) * pw[l <= tr ? 3 * (tr - l) : 0];
        }
        if (ok) st4_split<SPLIT>(Wms, Wmls, Cfg::LDC, tr, j0 + 4 * gq, x);
      });
      __syncthreads();
      // O = diag(g^(3(tau+1))) Q W0' + Wm Y
      for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        f32x4 x = pt2y<SPLIT, false, false, DK>(zero4(), Qs, Cfg::LDQ, Ws, Wls, Cfg::LDV, i0, j0, lane);
        x *= pw[3 * (i0 + nn + 1)];
        x = pt2x<SPLIT, false, false, BC>(x, Wms, Wmls, Cfg::LDC, Ys, Cfg::LDV, i0, j0, lane);
        O[it] = x;
        if (NORM && ok && j0 + 4 * gq == DV) dens[i0 + nn] = x[0];
      });
    } else {
      // segment maps: weights relative to the segment end (L = seglen tokens, u = u0 + tau)
      const int u0 = ch * BC;
      const float bq = exp2f(a.log2g * (float)(3 * seglen - u0 - BC));
      const float bx = exp2f(a.log2g * (float)(3 * seglen - 2 * u0 - 2 * BC));
      for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
        Q2[it] = ptw<true, false, BC>(Q2[it], Qs, Cfg::LDQ, Qs, Cfg::LDQ, i0, j0, lane,
                                      [&](int t) { return bq * pw[BC - 1 - t]; });
        X2[it] = ptw<true, false, BC>(X2[it], Zs, Cfg::LDQ, Qs, Cfg::LDQ, i0, j0, lane,
                                      [&](int t) { return bx * pw[2 * (BC - 1 - t)]; });
      });
      for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
        X1[it] = ptw<true, false, BC>(X1[it], Qs, Cfg::LDQ, Ys, Cfg::LDV, i0, j0, lane,
                                      [&](int t) { return bx * pw[2 * (BC - 1 - t)]; });
      });
    }
    // state updates
    const float gB = pw[BC], gB3 = pw[3 * BC];
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
      S[it] = ptw<true, false, BC>(gB * S[it], Ks, Cfg::LDQ, Ks, Cfg::LDQ, i0, j0, lane,
                                   [&](int i) { return pw[BC - 1 - i]; });
    });
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
      P[it] = ptw<true, false, BC>(gB * P[it], Ks, Cfg::LDQ, Vs, Cfg::LDV, i0, j0, lane,
                                   [&](int i) { return pw[BC - 1 - i]; });
      W[it] = ptw<true, false, BC>(gB3 * W[it], Zs, Cfg::LDQ, Ys, Cfg::LDV, i0, j0, lane,
                                   [&](int l) { return pw[3 * (BC - 1 - l)]; });
    });
    __syncthreads();  // dens complete; every read of this chunk's LDS done
    if constexpr (OUT) {
      T *oh = (T *)a.out + hv;
      for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int it) {
        const int tr = i0 + nn;
        f32x4 x = O[it];
        if (NORM && a.normalize) x *= 1.f / dens[tr];
        if (ok) st_out(oh, a.dv, t0 + tr, j0 + 4 * gq, a.n, x);
      });
      if (NORM && a.den_out && tid < BC && t0 + tid < a.n) a.den_out[(long)bh * a.n + t0 + tid] = dens[tid];
    }
  }
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * (a.nseg - 1) + seg) * Cfg::SB;
    float *sQ2 = sb + Cfg::PB, *sX1 = sQ2 + DK * DK, *sX2 = sX1 + DK * DVP;
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int it) {
      const int o = (i0 + nn) * DK + j0 + 4 * gq;
      if (ok) {
        *(f32x4 *)(sb + o) = S[it];
        *(f32x4 *)(sQ2 + o) = Q2[it];
        *(f32x4 *)(sX2 + o) = X2[it];
      }
    });
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      const int o = (i0 + nn) * DVP + j0 + 4 * gq;
      if (ok) {
        *(f32x4 *)(sb + DK * DK + o) = P[it];
        *(f32x4 *)(sb + DK * DK + DK * DVP + o) = W[it];
        *(f32x4 *)(sX1 + o) = X1[it];
      }
    });
  }
  if constexpr (OUT && LEAD) {
    // the state after segment 0 is the prefix S | P' | W' of segment 1 (the layout it is read in)
    float *pb = a.prefix + ((long)bh * a.nseg + seg + 1) * Cfg::PB;
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) *(f32x4 *)(pb + (i0 + nn) * DK + j0 + 4 * gq) = S[it];
    });
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      const int o = (i0 + nn) * DVP + j0 + 4 * gq;
      if (ok) {
        *(f32x4 *)(pb + DK * DK + o) = P[it];
        *(f32x4 *)(pb + DK * DK + DK * DVP + o) = W[it];
      }
    });
  }
}

// Walks segments (OUT ? seg_lo .. nseg-1 : 0 .. nseg-2) of every head, one workgroup each.
template <typename T, int DK, int DV, int DVP, int BC, bool OUT, bool NORM>
__global__ void __launch_bounds__(BWD_THREADS) ho3_walk_kernel(Ho3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[ho3_lds_bytes<T, DK, DVP, BC, ho3_split<T, NORM>()>()];
  const int lo = OUT ? a.seg_lo : 0, nr = (OUT ? a.nseg : a.nseg - 1) - lo;
  ho3_walk_body<T, DK, DV, DVP, BC, OUT, NORM, false>(a, blockIdx.x / nr, lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head for its outputs and
// leave the prefix of segment 1; the rest summarise segments 1 .. nseg-2 of every head.
template <typename T, int DK, int DV, int DVP, int BC, bool NORM>
__global__ void __launch_bounds__(BWD_THREADS) ho3_lead_kernel(Ho3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[ho3_lds_bytes<T, DK, DVP, BC, ho3_split<T, NORM>()>()];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    ho3_walk_body<T, DK, DV, DVP, BC, true, NORM, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = a.nseg - 2;
    ho3_walk_body<T, DK, DV, DVP, BC, false, NORM, false>(a, i / nr, 1 + i % nr, lds);
  }
}

// Exclusive scan over segments (the fold of each full segment into the running
// state), per (b, h), fp32 on VALU.  Workgroup (bh, sp) owns rows 16 sp ..
// 16 sp + 15 of S and W' (the fold of a row needs only that row of S, of X2
// and of S Q2, plus all of P' and X1); every workgroup of a head keeps the
// whole P' sequence in LDS (elementwise), so the workgroups never wait on
// each other.  Each writes its rows of every prefix.
template <int DK, int DVP>
__global__ void __launch_bounds__(256) ho3_scan_kernel(Ho3Args a, float G) {
  constexpr long PB = (long)DK * DK + 2L * DK * DVP, SB = PB + 2L * DK * DK + (long)DK * DVP;
  // a thread owns 4 consecutive columns of a row (reads of P', X1, Q2 as float4: 4 FMAs each)
  constexpr int WQ = 16 * DVP / 4, NWQ = (WQ + 255) / 256;  // 4-column groups of the W' rows
  constexpr int TQ = 16 * DK / 4, NTQ = (TQ + 255) / 256;   // of the S Q2 rows
  __shared__ __attribute__((aligned(16))) float Pl[DK * DVP], Sl[16 * DK], Tl[16 * DK], Ql[DK * DK], Xl[DK * DVP];
  const int tid = threadIdx.x, bh = blockIdx.x, sp = blockIdx.y, r0 = 16 * sp;
  const float G3 = G * G * G;
  float *pre = a.prefix + (long)bh * a.nseg * PB;
  const int rs = a.first;  // 1: the prefix of segment 1 is given (written by segment 0's walk)
  const float *given = pre + (long)rs * PB;
  for (int e = 4 * tid; e < DK * DVP; e += 1024)
    *(f32x4 *)(Pl + e) = rs ? *(const f32x4 *)(given + DK * DK + e) : zero4();
  for (int e = 4 * tid; e < 16 * DK; e += 1024)
    *(f32x4 *)(Sl + e) = rs ? *(const f32x4 *)(given + r0 * DK + e) : zero4();
  f32x4 W[NWQ];  // W'[r0 + f][c0 .. c0 + 3] for group q = tid + 256 i: f = q / (DVP/4), c0 = 4 (q % (DVP/4))
#pragma unroll
  for (int i = 0; i < NWQ; ++i) {
    const int q = tid + 256 * i;
    const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
    W[i] = (rs && (WQ % 256 == 0 || q < WQ)) ? *(const f32x4 *)(given + DK * DK + DK * DVP + (r0 + f) * DVP + c0)
                                             : zero4();
  }
  for (int r = rs; r < a.nseg; ++r) {
    float *pr = pre + (long)r * PB;
    const bool put = r > rs || rs == 0;  // a given prefix is already in place
    __syncthreads();  // Pl, Sl hold the state before segment r
    if (put)
      for (int e = tid; e < 16 * DK; e += 256) pr[r0 * DK + e] = Sl[e];
#pragma unroll
    for (int i = 0; i < NWQ; ++i) {
      const int q = tid + 256 * i;
      if (put && (WQ % 256 == 0 || q < WQ)) {
        const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
        *(f32x4 *)(pr + DK * DK + (r0 + f) * DVP + c0) = *(const f32x4 *)(Pl + (r0 + f) * DVP + c0);
        *(f32x4 *)(pr + DK * DK + DK * DVP + (r0 + f) * DVP + c0) = W[i];
      }
    }
    if (r == a.nseg - 1) break;
    const float *sb = a.sums + ((long)bh * (a.nseg - 1) + r) * SB;
    const float *Q2 = sb + PB, *X1 = Q2 + DK * DK, *X2 = X1 + DK * DVP;
    for (int e = 4 * tid; e < DK * DK; e += 1024) *(f32x4 *)(Ql + e) = *(const f32x4 *)(Q2 + e);  // the maps, staged
    for (int e = 4 * tid; e < DK * DVP; e += 1024) *(f32x4 *)(Xl + e) = *(const f32x4 *)(X1 + e);
    __syncthreads();
    // T = S Q2 + X2 for the group's rows
#pragma unroll
    for (int i = 0; i < NTQ; ++i) {
      const int q = tid + 256 * i;
      if (TQ % 256 == 0 || q < TQ) {
        const int f = q / (DK / 4), c0 = 4 * (q % (DK / 4));
        f32x4 t = *(const f32x4 *)(X2 + (r0 + f) * DK + c0);
        for (int b = 0; b < DK; ++b) t += Sl[f * DK + b] * *(const f32x4 *)(Ql + b * DK + c0);
        *(f32x4 *)(Tl + f * DK + c0) = t;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NWQ; ++i) {
      const int q = tid + 256 * i;
      if (WQ % 256 == 0 || q < WQ) {
        const int f = q / (DVP / 4), c0 = 4 * (q % (DVP / 4));
        f32x4 acc = zero4();
        for (int b = 0; b < DK; ++b)
          acc += Tl[f * DK + b] * *(const f32x4 *)(Pl + b * DVP + c0) + Sl[f * DK + b] * *(const f32x4 *)(Xl + b * DVP + c0);
        W[i] = G3 * W[i] + *(const f32x4 *)(sb + DK * DK + DK * DVP + (r0 + f) * DVP + c0) + acc;
      }
    }
    __syncthreads();  // every read of the state before segment r done
    for (int e = 4 * tid; e < DK * DVP; e += 1024)
      *(f32x4 *)(Pl + e) = G * *(const f32x4 *)(Pl + e) + *(const f32x4 *)(sb + DK * DK + e);
    for (int e = tid; e < 16 * DK; e += 256) Sl[e] = G * Sl[e] + sb[r0 * DK + e];
  }
}

template <typename T, int DK, int DV, bool NORM>
static hipError_t launch_ho3_t(int phase, int BH, const Ho3Args &a, float gseg, hipStream_t s) {
  constexpr int DVP = lds_walk_dvp(sizeof(T) == 4, DV, NORM);
  // d <= 64 here.  Under the ratio at dv = 128 the state is 160 columns wide (P', W'), and 64-token
  // chunks spilled about 100 registers to scratch per wave; 32-token chunks halve the chunk-sized tiles
  // and keep the walk in registers (decay workload's shape with the ratio: 1.94 -> 0.78 ms).  At dv = 64
  // the 64-token chunk is faster.
  constexpr int BC = (NORM && DVP > 128) ? 32 : lds_walk_chunk(sizeof(T) == 4, DK);
  switch (phase) {
    case HO3_SUMMARY:
      hipLaunchKernelGGL((ho3_walk_kernel<T, DK, DV, DVP, BC, false, NORM>), dim3(BH * (a.nseg - 1)),
                         dim3(BWD_THREADS), 0, s, a);
      return hipGetLastError();
    case HO3_SCAN:
      hipLaunchKernelGGL((ho3_scan_kernel<DK, DVP>), dim3(BH, DK / 16), dim3(256), 0, s, a, gseg);
      return hipGetLastError();
    case HO3_OUTPUT:
      hipLaunchKernelGGL((ho3_walk_kernel<T, DK, DV, DVP, BC, true, NORM>), dim3(BH * (a.nseg - a.seg_lo)),
                         dim3(BWD_THREADS), 0, s, a);
      return hipGetLastError();
    case HO3_LEAD:
      if (a.nseg < 2 || a.nbh != BH) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ho3_lead_kernel<T, DK, DV, DVP, BC, NORM>), dim3(BH * (a.nseg - 1)), dim3(BWD_THREADS),
                         0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK, int DV>
static hipError_t launch_ho3_n(bool norm, int phase, int BH, const Ho3Args &a, float gseg, hipStream_t s) {
  return norm ? launch_ho3_t<T, DK, DV, true>(phase, BH, a, gseg, s)
              : launch_ho3_t<T, DK, DV, false>(phase, BH, a, gseg, s);
}


hipError_t launch_ho3(int dtype, int DK, int DV, bool norm, int phase, int BH, const Ho3Args &a, float gseg,
                      hipStream_t s) {
  if (dtype == 0) {
    if (DK == 16 && DV == 16) return launch_ho3_n<float, 16, 16>(norm, phase, BH, a, gseg, s);
    if (DK == 64 && DV == 64) return launch_ho3_n<float, 64, 64>(norm, phase, BH, a, gseg, s);
    return hipErrorInvalidValue;
  }
  if (DK == 64 && DV == 64) return launch_ho3_n<bf16, 64, 64>(norm, phase, BH, a, gseg, s);
  // without den the walks at d <= 64, dv > 64 run on the register-resident walker; the scan
  // between them is the same
  if (DK == 64 && DV == 128 && !norm && phase != HO3_SCAN) return launch_ho38(phase, BH, a, s);
  if (DK == 64 && DV == 128) return launch_ho3_n<bf16, 64, 128>(norm, phase, BH, a, gseg, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
