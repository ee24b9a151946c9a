// hla2_bwd.h -- chunk walkers of the backward pass: the gradients of the
// masked second-order HLA forward with respect to q, k and v.
//
// The pages train through the scan (technical summary of arXiv 2510.27258 on
// gist.science, §4) but print no gradient, so these kernels run the adjoint of
// the chunked forward, derived by the chain rule.  With U' = [SC - G | Sm - h]
// (the corrected state, one column per value plus one for the denominator),
// v' = [v | 1] and g' the upstream gradient of [num | den], the forward and its
// adjoint per token are
//   S_t = g S_{t-1} + k k^T,   z_t = S_t q_t,   U'_t = g^2 U'_{t-1} + z_t v'^T,
//   Ubar_t = q_t g'^T + g^2 Ubar_{t+1},  zbar_t = Ubar_t v'_t,
//   Shat_t = zbar_t q_t^T + q_t zbar_t^T + g Shat_{t+1}          (Shat = Sbar + Sbar^T)
//   dq_t = U'_t g'_t + S_t zbar_t,  dv_t = Ubar_t^T z_t,  dk_t = Shat_t k_t.
// Per chunk of BC tokens (local index tau, lower triangles include the
// diagonal, D1[t][i] = g^(t-i), D2 = D1 o D1), from the forward state (S0, U0')
// at the chunk start and the adjoint state (Ubar, Shat) at the chunk end:
//   Ad = L o D1 o (Q K^T),  Bm = L o D2 o (G' V'^T),
//   Z  = diag(g^(tau+1)) Q S0 + Ad K,
//   Zb = Bm^T Q + diag(g^(2(BC-tau))) V' Ubar^T,
//   W  = L o D2 o (Q Z^T),  Ek = L o D1 o (Zb K^T),
//   dV' = W^T G' + diag(g^(2(BC-tau))) Z Ubar,
//   dQ  = diag(g^(tau+1)) [diag(g^(tau+1)) G' U0'^T + Zb S0] + Bm Z + Ek K,
//   dK  = Ad^T Zb + Ek^T Q + diag(g^(BC-tau)) K Shat,
// and the states move on as
//   S   <- g^BC S + K^T diag(g^(BC-1-i)) K,   U' <- g^(2BC) U' + Z^T diag(g^(2(BC-1-tau))) V',
//   Ubar <- g^(2BC) Ubar + Q^T diag(g^(2 tau)) G',
//   Shat <- g^BC Shat + Zb^T diag(g^tau) Q + Q^T diag(g^tau) Zb.
// Tokens past the end are zero rows in Q, K, V' (its ones column too) and G',
// so a ragged last chunk takes the same path.
//
// Kernels:
//   bwd_pre_kernel     one launch with two roles, 4 waves per workgroup:
//                      for every (b, h, segment) it walks the segment forwards
//                      from its scanned prefix and writes every chunk's
//                      (S0, U0') in the element type; for every (b, h, segment
//                      >= 1) it walks the segment backwards from a zero adjoint
//                      state and writes its adjoint summary (Ubar, Shat).  Each
//                      role has a compact LDS layout, so two workgroups share a
//                      CU and the two roles run side by side;
//   bwd_walk_kernel    8 waves per (b, h, segment): walks the segment backwards
//                      from its scanned adjoint state, reads the stored forward
//                      states (fetched a chunk phase ahead) and writes dq, dk, dv.
// Every product is a set of 16x16 MFMA tiles computed transposed, so that a
// lane holds four consecutive columns of one row of the result; the waves of
// a workgroup take the tiles in turn.  Tile loops have compile-time trip counts,
// and a wave with no tile left repeats the last one without storing it.  The
// only MFMAs under a (wave-uniform) branch are those of the C x C tiles that the
// causal mask zeroes whole, which are skipped (for_causal_tiles); products that
// contract over such a matrix skip the k-tiles outside its triangle (pt_tri).
#pragma once
#include "hla2_internal.h"
#include "hla2_tiles.h"

namespace hla2 {

// LDS layouts.  Row pitches carry lds_pad_bytes<T>() of padding, except in the adjoint-summary
// role of the two-role pre-walk, which keeps 16 bytes so that two of its workgroups share a CU.
constexpr int RSUM_PADB = 16;
template <typename T, int DK, int DVP, int BC, int PADB = lds_pad_bytes<T>()>
struct BwdPitch {
  static constexpr int PAD = PADB / sizeof(T);
  static constexpr int LDQ = DK + PAD;   // Q, K, Z, Zb rows; S / Shat copy rows
  static constexpr int LDV = DVP + PAD;  // V', G' rows; Ubar copy rows
  static constexpr int LDC = BC + PAD;   // BC x BC masks
  static constexpr int BLOCK = DK * DK + DK * DVP;  // stored chunk state S0 | U0' (elements)
};
// gradient walk: everything
template <typename T, int DK, int DVP, int BC>
struct BwdCfg : BwdPitch<T, DK, DVP, BC> {
  using P = BwdPitch<T, DK, DVP, BC>;
  static constexpr int Q_OFF = 0, K_OFF = Q_OFF + BC * P::LDQ, V_OFF = K_OFF + BC * P::LDQ,
                       G_OFF = V_OFF + BC * P::LDV, U_OFF = G_OFF + BC * P::LDV, S_OFF = U_OFF + DK * P::LDV,
                       AD_OFF = S_OFF + DK * P::LDQ, BM_OFF = AD_OFF + BC * P::LDC, W_OFF = BM_OFF + BC * P::LDC,
                       EK_OFF = W_OFF + BC * P::LDC, Z_OFF = EK_OFF + BC * P::LDC, ZB_OFF = Z_OFF + BC * P::LDQ,
                       QT_OFF = ZB_OFF + BC * P::LDQ;
  // at d <= 64 the rows of Q~ = diag(g^tau) Q follow (the Shat update's weighted operand)
  static constexpr bool QT = DK <= 64;
  static constexpr int ELEMS = QT_OFF + (QT ? BC * P::LDQ : 0);
};
// forward-state walk: Q, K, V', the S copy, Ad, Z
template <typename T, int DK, int DVP, int BC>
struct StateLay : BwdPitch<T, DK, DVP, BC> {
  using P = BwdPitch<T, DK, DVP, BC>;
  static constexpr int Q_OFF = 0, K_OFF = BC * P::LDQ, V_OFF = K_OFF + BC * P::LDQ, S_OFF = V_OFF + BC * P::LDV,
                       AD_OFF = S_OFF + DK * P::LDQ, Z_OFF = AD_OFF + BC * P::LDC, ELEMS = Z_OFF + BC * P::LDQ;
};
// adjoint-summary walk: Q, V', G', the Ubar copy, Bm, Zb
template <typename T, int DK, int DVP, int BC>
struct RsumLay : BwdPitch<T, DK, DVP, BC, RSUM_PADB> {
  using P = BwdPitch<T, DK, DVP, BC, RSUM_PADB>;
  static constexpr int Q_OFF = 0, V_OFF = BC * P::LDQ, G_OFF = V_OFF + BC * P::LDV, U_OFF = G_OFF + BC * P::LDV,
                       BM_OFF = U_OFF + DK * P::LDV, ZB_OFF = BM_OFF + BC * P::LDC, ELEMS = ZB_OFF + BC * P::LDQ;
};
constexpr int BWD_PRE_WAVES = 4, BWD_PRE_THREADS = 64 * BWD_PRE_WAVES;

// ---------------------------------------------------------------------------
// Forward state of every chunk of one segment: S0 and U0' at the chunk start,
// in the element type (the precision the gradient kernel's products consume).
// part: -1 the whole segment; with a split segment 0 (half0 > 0), 0 its first half (from the zero
// state) and 1 its second half, which starts from the forward summary of the first (fsum block 0:
// S | C | U | m | u; the state of a segment that starts from zero is its summary).
template <typename T, int DK, int DV, int DVP, int BC, bool NORM, int NW>
__device__ __forceinline__ void bwd_state_body(const BwdArgs &a, T *smem, const float *pw, int bh, int seg,
                                               int part = -1) {
  using L = StateLay<T, DK, DVP, BC>;
  constexpr int NTH = 64 * NW;
  T *const Qs = smem + L::Q_OFF, *const Ks = smem + L::K_OFF, *const Vs = smem + L::V_OFF;
  T *const Ss = smem + L::S_OFF, *const Ads = smem + L::AD_OFF, *const Zs = smem + L::Z_OFF;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, nn = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tok0 = seg * a.cps * a.kc, tokE = min(a.n, tok0 + a.cps * a.kc);
  if (part == 0) tokE = a.half0 * a.kc;
  if (part == 1) tok0 = a.half0 * a.kc;
  const int nch = (tokE - tok0 + BC - 1) / BC, c0 = tok0 / BC;
  const T *qh = (const T *)a.q + (long)bh * a.n * a.d, *kh = (const T *)a.k + (long)bh * a.n * a.d;
  const T *vh = (const T *)a.v + (long)bh * a.n * a.dv;
  T *cst = (T *)a.cstate + ((long)bh * a.nbc + c0) * L::BLOCK;

  f32x4 S[TileCount<DK, DK, NW>::PER], U[TileCount<DK, DVP, NW>::PER];
  // incoming state: the scanned prefix (S | U | u), the first half's summary (S | C | U | m | u) for
  // a second half, or zero for the first segment
  const float *pref = nullptr, *pU = nullptr, *pu = nullptr;
  if (part == 1) {
    pref = a.fsum + (long)bh * 2 * sum_block_floats(DK, DV);
    pU = pref + DK * DK + DK * DV;
    pu = pU + DK * DV + DK;
  } else if (a.prefix && seg > 0) {
    pref = a.prefix + ((long)bh * a.nseg + seg) * prefix_block_floats(DK, DV);
    pU = pref + DK * DK;
    pu = pU + DK * DV;
  }
  for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool, int it) {
    S[it] = pref ? *(const f32x4 *)(pref + (i0 + nn) * DK + j0 + 4 * gq) : zero4();
  });
  for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool, int it) {
    f32x4 x = zero4();
    if (pref) {
      const int r = i0 + nn, c = j0 + 4 * gq;
      if (c < DV) x = *(const f32x4 *)(pU + r * DV + c);
      else if (NORM && c == DV) x[0] = pu[r];
    }
    U[it] = x;
  });
  RowTile<T, BC, DK, NTH> rq, rk;
  RowTile<T, BC, DVP, NTH> rv;
  rq.fetch(qh, a.d, tok0, a.n, -1, tid);
  rk.fetch(kh, a.d, tok0, a.n, -1, tid);
  rv.fetch(vh, a.dv, tok0, a.n, NORM ? DV : -1, tid);

  for (int ch = 0; ch < nch; ++ch) {
    // state at the chunk start: a copy of S into LDS, and both into the chunk store (in the LDS
    // row layout, swizzle included, so the gradient walk reads its fragments with ld_rows_l)
    T *blk = cst + (long)ch * L::BLOCK;
    for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) {
        st4l(Ss, L::LDQ, i0 + nn, j0 + 4 * gq, S[it]);
        st4g(blk + (i0 + nn) * DK + (pcol<T>(j0 + 4 * gq) ^ tsw<T>(i0 + nn, DK)), S[it]);
      }
    });
    for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) st4g(blk + DK * DK + (i0 + nn) * DVP + (pcol<T>(j0 + 4 * gq) ^ tsw<T>(i0 + nn, DVP)), U[it]);
    });
    rq.put(Qs, L::LDQ, tid);
    rk.put(Ks, L::LDQ, tid);
    rv.put(Vs, L::LDV, tid);
    __syncthreads();
    {  // the next chunk's rows fly while this one is processed
      const int tn = tok0 + min(ch + 1, nch - 1) * BC;
      rq.fetch(qh, a.d, tn, a.n, -1, tid);
      rk.fetch(kh, a.d, tn, a.n, -1, tid);
      rv.fetch(vh, a.dv, tn, a.n, NORM ? DV : -1, tid);
    }
    // Ad = L o D1 o (Q K^T)
    for_tiles<BC, BC, NW>(w, [&](int i0, int j0, bool ok, int) {
      f32x4 x = pt<false, true, DK>(zero4(), Qs, L::LDQ, Ks, L::LDQ, i0, j0, lane);
      const int tr = i0 + nn;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ti = j0 + 4 * gq + e;
        // the factor is read and applied on every lane (clamped index, masked value) so
        // that no branch forms around the table read
        x[e] = (ti <= tr ? x[e] : 0.f) * pw[ti <= tr ? tr - ti : 0];
      }
      if (ok) st4l(Ads, L::LDC, tr, j0 + 4 * gq, x);
    });
    __syncthreads();
    // Z = diag(g^(tau+1)) Q S0 + Ad K
    for_tiles<BC, DK, NW>(w, [&](int i0, int j0, bool ok, int it) {
      f32x4 x = pt<false, true, DK>(zero4(), Qs, L::LDQ, Ss, L::LDQ, i0, j0, lane);
      x *= pw[i0 + nn + 1];
      x = pt_tri<false, false, BC>(x, Ads, L::LDC, Ks, L::LDQ, i0, j0, lane, tile_rows_lo<BC, DK, NW>(it),
                                   tile_rows_hi<BC, DK, NW>(it));
      if (ok) st4l(Zs, L::LDQ, i0 + nn, j0 + 4 * gq, x);
    });
    __syncthreads();
    // S <- g^BC S + K^T diag(g^(BC-1-i)) K;  U' <- g^(2BC) U' + Z^T diag(g^(2(BC-1-tau))) V'
    const float gB = pw[BC], gB2 = pw[2 * BC];
    for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool, int it) {
      S[it] = ptw<true, false, BC>(gB * S[it], Ks, L::LDQ, Ks, L::LDQ, i0, j0, lane,
                                   [&](int i) { return pw[BC - 1 - i]; });
    });
    for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool, int it) {
      U[it] = ptw<true, false, BC>(gB2 * U[it], Zs, L::LDQ, Vs, L::LDV, i0, j0, lane,
                                   [&](int t) { return pw[2 * (BC - 1 - t)]; });
    });
    __syncthreads();  // every read of Ss, Qs, Ks, Vs, Zs done before the next chunk overwrites them
  }
}

// ---------------------------------------------------------------------------
// Shared adjoint step: Bm, Zb into LDS (needs Q, V', G' and the Ubar copy).
template <typename T, int DK, int DVP, int BC, int NW, typename Lay>
__device__ __forceinline__ void bwd_bm_zb(T *smem, const float *pw, int w, int lane) {
  T *const Qs = smem + Lay::Q_OFF, *const Vs = smem + Lay::V_OFF, *const Gs = smem + Lay::G_OFF;
  T *const Ubs = smem + Lay::U_OFF, *const Bms = smem + Lay::BM_OFF, *const Zbs = smem + Lay::ZB_OFF;
  const int gq = lane >> 4, nn = lane & 15;
  // Bm = L o D2 o (G' V'^T)   (rows s, columns tau <= s)
  for_causal_tiles<BC, NW>(w, [&](int i0, int j0, bool ok, bool live) {
    f32x4 x = zero4();
    if (live) x = pt<false, true, DVP>(x, Gs, Lay::LDV, Vs, Lay::LDV, i0, j0, lane);
    const int s = i0 + nn;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tau = j0 + 4 * gq + e;
      // the factor is read and applied on every lane (clamped index, masked value) so
      // that no branch forms around the table read
      x[e] = (tau <= s ? x[e] : 0.f) * pw[tau <= s ? 2 * (s - tau) : 0];
    }
    if (ok) st4l(Bms, Lay::LDC, s, j0 + 4 * gq, x);
  });
  __syncthreads();
  // Zb = Bm^T Q + diag(g^(2(BC-tau))) V' Ubar^T
  for_tiles<BC, DK, NW>(w, [&](int i0, int j0, bool ok, int it) {
    f32x4 x = pt<false, true, DVP>(zero4(), Vs, Lay::LDV, Ubs, Lay::LDV, i0, j0, lane);
    x *= pw[2 * (BC - (i0 + nn))];
    x = pt_tri<true, false, BC>(x, Bms, Lay::LDC, Qs, Lay::LDQ, i0, j0, lane, tile_rows_lo<BC, DK, NW>(it),
                                tile_rows_hi<BC, DK, NW>(it));
    if (ok) st4l(Zbs, Lay::LDQ, i0 + nn, j0 + 4 * gq, x);
  });
}

// Adjoint state update (registers): Ubar <- g^(2BC) Ubar + Q^T diag(g^(2tau)) G';
// Shat <- g^BC Shat + Zb^T diag(g^tau) Q + Q^T diag(g^tau) Zb.  With QT the layout holds
// Q~ = diag(g^tau) Q as well, and the Shat update reads it instead of weighting fragments.
template <typename T, int DK, int DVP, int BC, int NW, typename Lay, bool QT = false>
__device__ __forceinline__ void bwd_adjoint_update(T *smem, const float *pw, int w, int lane, f32x4 *Ub, f32x4 *Sh) {
  T *const Qs = smem + Lay::Q_OFF, *const Gs = smem + Lay::G_OFF, *const Zbs = smem + Lay::ZB_OFF;
  const float gB = pw[BC], gB2 = pw[2 * BC];
  for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool, int it) {
    Ub[it] = ptw<true, false, BC>(gB2 * Ub[it], Qs, Lay::LDQ, Gs, Lay::LDV, i0, j0, lane,
                                  [&](int s) { return pw[2 * s]; });
  });
  if constexpr (QT) {
    T *const Qts = smem + Lay::QT_OFF;
    for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool, int it) {
      f32x4 x = pt<true, false, BC>(gB * Sh[it], Zbs, Lay::LDQ, Qts, Lay::LDQ, i0, j0, lane);
      Sh[it] = pt<true, false, BC>(x, Qts, Lay::LDQ, Zbs, Lay::LDQ, i0, j0, lane);
    });
  } else {
    for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool, int it) {
      f32x4 x = ptw<true, false, BC>(gB * Sh[it], Zbs, Lay::LDQ, Qs, Lay::LDQ, i0, j0, lane,
                                     [&](int s) { return pw[s]; });
      Sh[it] = ptw<true, false, BC>(x, Qs, Lay::LDQ, Zbs, Lay::LDQ, i0, j0, lane, [&](int s) { return pw[s]; });
    });
  }
}

// copies of the adjoint state for the next chunk's products (Shat only where read)
template <typename T, int DK, int DVP, int NW, bool WITH_S, typename Lay>
__device__ __forceinline__ void bwd_adjoint_copy(T *smem, int w, int lane, const f32x4 *Ub, const f32x4 *Sh) {
  const int gq = lane >> 4, nn = lane & 15;
  T *const Ubs = smem + Lay::U_OFF;
  for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool ok, int it) {
    if (ok) st4l(Ubs, Lay::LDV, i0 + nn, j0 + 4 * gq, Ub[it]);
  });
  if constexpr (WITH_S) {
    T *const Shs = smem + Lay::S_OFF;
    for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool ok, int it) {
      if (ok) st4l(Shs, Lay::LDQ, i0 + nn, j0 + 4 * gq, Sh[it]);
    });
  }
}

// ---------------------------------------------------------------------------
// Adjoint summary of a segment (segments 1 .. nseg-1): walked backwards from a
// zero adjoint state at the segment end.
template <typename T, int DK, int DV, int DVP, int BC, bool NORM, int NW>
__device__ __forceinline__ void bwd_rsum_body(const BwdArgs &a, T *smem, const float *pw, int bh, int seg) {
  using L = RsumLay<T, DK, DVP, BC>;
  constexpr int NTH = 64 * NW;
  T *const Qs = smem + L::Q_OFF, *const Vs = smem + L::V_OFF, *const Gs = smem + L::G_OFF;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, nn = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = seg * a.cps * a.kc, tokE = min(a.n, tok0 + a.cps * a.kc);
  const int nch = (tokE - tok0 + BC - 1) / BC;
  const T *qh = (const T *)a.q + (long)bh * a.n * a.d, *vh = (const T *)a.v + (long)bh * a.n * a.dv;
  const T *gh = (const T *)a.g + (long)bh * a.n * a.gld;
  f32x4 Ub[TileCount<DK, DVP, NW>::PER], Sh[TileCount<DK, DK, NW>::PER];
#pragma unroll
  for (int i = 0; i < TileCount<DK, DVP, NW>::PER; ++i) Ub[i] = zero4();
#pragma unroll
  for (int i = 0; i < TileCount<DK, DK, NW>::PER; ++i) Sh[i] = zero4();
  bwd_adjoint_copy<T, DK, DVP, NW, false, L>(smem, w, lane, Ub, Sh);
  RowTile<T, BC, DK, NTH> rq;
  RowTile<T, BC, DVP, NTH> rv, rg;
  {
    const int t0 = tok0 + (nch - 1) * BC;
    rq.fetch(qh, a.d, t0, a.n, -1, tid);
    rv.fetch(vh, a.dv, t0, a.n, NORM ? DV : -1, tid);
    rg.fetch(gh, a.gld, t0, a.n, -1, tid);
  }

  for (int ch = nch - 1; ch >= 0; --ch) {
    rq.put(Qs, L::LDQ, tid);
    rv.put(Vs, L::LDV, tid);
    rg.put(Gs, L::LDV, tid);
    __syncthreads();
    {  // the next (earlier) chunk's rows fly while this one is processed
      const int tn = tok0 + max(ch - 1, 0) * BC;
      rq.fetch(qh, a.d, tn, a.n, -1, tid);
      rv.fetch(vh, a.dv, tn, a.n, NORM ? DV : -1, tid);
      rg.fetch(gh, a.gld, tn, a.n, -1, tid);
    }
    bwd_bm_zb<T, DK, DVP, BC, NW, L>(smem, pw, w, lane);
    __syncthreads();
    bwd_adjoint_update<T, DK, DVP, BC, NW, L>(smem, pw, w, lane, Ub, Sh);
    __syncthreads();  // reads of the old copies and of the chunk done
    bwd_adjoint_copy<T, DK, DVP, NW, false, L>(smem, w, lane, Ub, Sh);
  }
  float *out = a.rsum + ((long)bh * a.nseg + seg) * ((long)DK * DVP + DK * DK);
  for_tiles<DK, DVP, NW>(w, [&](int i0, int j0, bool ok, int it) {
    if (ok) *(f32x4 *)(out + (i0 + nn) * DVP + j0 + 4 * gq) = Ub[it];
  });
  for_tiles<DK, DK, NW>(w, [&](int i0, int j0, bool ok, int it) {
    if (ok) *(f32x4 *)(out + DK * DVP + (i0 + nn) * DK + j0 + 4 * gq) = Sh[it];
  });
}

// Both roles in one launch: workgroups 0 .. BH*nseg-1 store the forward states of
// segment (bh, seg); the rest form the adjoint summaries of segments 1 .. nseg-1.
// MINW: waves per SIMD the register allocation must leave room for (2 where two
// workgroups fit a CU's LDS and their registers fit without spilling: d <= 64).
template <typename T, int DK, int DV, int DVP, int BC, bool NORM, int MINW>
__global__ void __launch_bounds__(BWD_PRE_THREADS, MINW) bwd_pre_kernel(BwdArgs a) {
  using SL = StateLay<T, DK, DVP, BC>;
  using RL = RsumLay<T, DK, DVP, BC>;
  constexpr int ELEMS = SL::ELEMS > RL::ELEMS ? SL::ELEMS : RL::ELEMS;
  __shared__ __attribute__((aligned(16))) T smem[ELEMS];
  __shared__ float pw[2 * BC + 3];
  for (int e = threadIdx.x; e < 2 * BC + 3; e += BWD_PRE_THREADS) pw[e] = exp2f((float)e * a.log2g);
  __syncthreads();
  const int b = blockIdx.x;
  // (d <= 64 only: at d = 128 the extra role copies would push the register allocation into spills)
  if (DK <= 64 && a.half0 > 0) {
    // two segments, segment 0's forward-state walk split in halves: the adjoint summaries and the
    // state walks of segment 1 first, then the halves of segment 0 (four workgroups per head, two
    // per CU, so that every CU gets a long walk and a short one)
    const int nb = a.nbh;
    if (b < nb) {
      bwd_rsum_body<T, DK, DV, DVP, BC, NORM, BWD_PRE_WAVES>(a, smem, pw, b, 1);
    } else if (b < 2 * nb) {
      bwd_state_body<T, DK, DV, DVP, BC, NORM, BWD_PRE_WAVES>(a, smem, pw, b - nb, 1);
    } else {
      const int i = b - 2 * nb;
      bwd_state_body<T, DK, DV, DVP, BC, NORM, BWD_PRE_WAVES>(a, smem, pw, i / 2, 0, i % 2);
    }
    return;
  }
  const int nstate = (int)(gridDim.x - (unsigned)(a.nbh * (a.nseg - 1)));
  if (b < nstate) {
    bwd_state_body<T, DK, DV, DVP, BC, NORM, BWD_PRE_WAVES>(a, smem, pw, b / a.nseg, b % a.nseg);
  } else {
    const int r = b - nstate;
    bwd_rsum_body<T, DK, DV, DVP, BC, NORM, BWD_PRE_WAVES>(a, smem, pw, r / (a.nseg - 1), 1 + r % (a.nseg - 1));
  }
}

// ---------------------------------------------------------------------------
// Gradients: each segment walked backwards from its scanned adjoint state.
template <typename T, int DK, int DV, int DVP, int BC, bool NORM>
__global__ void __launch_bounds__(BWD_THREADS) bwd_walk_kernel(BwdArgs a) {
  using Cfg = BwdCfg<T, DK, DVP, BC>;
  constexpr int NW = BWD_WAVES, KT = Ktile<T>::ROWS;
  typedef typename Ktile<T>::frag Frag;
  __shared__ __attribute__((aligned(16))) T smem[Cfg::ELEMS];
  __shared__ float pw[2 * BC + 3];
  T *const Qs = smem + Cfg::Q_OFF, *const Ks = smem + Cfg::K_OFF, *const Vs = smem + Cfg::V_OFF;
  T *const Gs = smem + Cfg::G_OFF, *const Ubs = smem + Cfg::U_OFF, *const Shs = smem + Cfg::S_OFF;
  T *const Ads = smem + Cfg::AD_OFF, *const Bms = smem + Cfg::BM_OFF, *const Ws = smem + Cfg::W_OFF;
  T *const Eks = smem + Cfg::EK_OFF, *const Zs = smem + Cfg::Z_OFF, *const Zbs = smem + Cfg::ZB_OFF;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, nn = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
  const int tok0 = seg * a.cps * a.kc, tokE = min(a.n, tok0 + a.cps * a.kc);
  const int nch = (tokE - tok0 + BC - 1) / BC, c0 = tok0 / BC;
  const long hq = (long)bh * a.n * a.d, hv = (long)bh * a.n * a.dv;
  const T *qh = (const T *)a.q + hq, *kh = (const T *)a.k + hq, *vh = (const T *)a.v + hv;
  const T *gh = (const T *)a.g + (long)bh * a.n * a.gld;
  T *dqh = (T *)a.dq_out + hq, *dkh = (T *)a.dk_out + hq, *dvh = (T *)a.dv_out + hv;
  const T *cst = (const T *)a.cstate + ((long)bh * a.nbc + c0) * Cfg::BLOCK;
  for (int e = tid; e < 2 * BC + 3; e += BWD_THREADS) pw[e] = exp2f((float)e * a.log2g);
  // the Z and dQ tiles of this wave all share one block of d columns (8 waves divide DK/16 evenly)
  const int jw = 16 * (w % (DK / 16));

  f32x4 Ub[TileCount<DK, DVP>::PER], Sh[TileCount<DK, DK>::PER];
  {
    const float *suf = a.suffix + ((long)bh * a.nseg + seg) * ((long)DK * DVP + DK * DK);
    for_tiles<DK, DVP>(w, [&](int i0, int j0, bool, int it) {
      Ub[it] = *(const f32x4 *)(suf + (i0 + nn) * DVP + j0 + 4 * gq);
    });
    for_tiles<DK, DK>(w, [&](int i0, int j0, bool, int it) {
      Sh[it] = *(const f32x4 *)(suf + DK * DVP + (i0 + nn) * DK + j0 + 4 * gq);
    });
  }
  bwd_adjoint_copy<T, DK, DVP, NW, true, Cfg>(smem, w, lane, Ub, Sh);
  RowTile<T, BC, DK> rq, rk;
  RowTile<T, BC, DVP> rv, rg;
  {
    const int t0 = tok0 + (nch - 1) * BC;
    rq.fetch(qh, a.d, t0, a.n, -1, tid);
    rk.fetch(kh, a.d, t0, a.n, -1, tid);
    rv.fetch(vh, a.dv, t0, a.n, NORM ? DV : -1, tid);
    rg.fetch(gh, a.gld, t0, a.n, -1, tid);
  }

  for (int ch = nch - 1; ch >= 0; --ch) {
    const int t0 = tok0 + ch * BC;
    // this chunk's stored forward state: the wave's S0 and U0' fragments, read now and
    // consumed after the Ad / Bm / Zb phase
    Frag s0f[DK / KT], u0f[DVP / KT];
    {
      const T *S0 = cst + (long)ch * Cfg::BLOCK, *U0 = S0 + DK * DK;
#pragma unroll
      for (int k = 0; k < DK / KT; ++k) s0f[k] = ld_rows_l(S0, DK, jw, k * KT, lane);
#pragma unroll
      for (int k = 0; k < DVP / KT; ++k) u0f[k] = ld_rows_l(U0, DVP, jw, k * KT, lane);
    }
    rq.put(Qs, Cfg::LDQ, tid);
    if constexpr (Cfg::QT) rq.put_scaled(smem + Cfg::QT_OFF, Cfg::LDQ, tid, a.log2g);  // Q~ = diag(g^tau) Q
    rk.put(Ks, Cfg::LDQ, tid);
    rv.put(Vs, Cfg::LDV, tid);
    rg.put(Gs, Cfg::LDV, tid);
    __syncthreads();
    {  // the next (earlier) chunk's rows fly while this one is processed
      const int tn = tok0 + max(ch - 1, 0) * BC;
      rq.fetch(qh, a.d, tn, a.n, -1, tid);
      rk.fetch(kh, a.d, tn, a.n, -1, tid);
      rv.fetch(vh, a.dv, tn, a.n, NORM ? DV : -1, tid);
      rg.fetch(gh, a.gld, tn, a.n, -1, tid);
    }
    // Ad = L o D1 o (Q K^T)
    for_causal_tiles<BC>(w, [&](int i0, int j0, bool ok, bool live) {
      f32x4 x = zero4();
      if (live) x = pt<false, true, DK>(x, Qs, Cfg::LDQ, Ks, Cfg::LDQ, i0, j0, lane);
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
    // Bm, then Zb (one barrier inside)
    bwd_bm_zb<T, DK, DVP, BC, NW, Cfg>(smem, pw, w, lane);
    // Z = diag(g^(tau+1)) Q S0 + Ad K   (Ad is complete: the barrier inside bwd_bm_zb)
    for_tiles<BC, DK>(w, [&](int i0, int j0, bool ok, int it) {
      f32x4 x = pt_frags<DK>(zero4(), s0f, Qs, Cfg::LDQ, i0, lane);
      x *= pw[i0 + nn + 1];
      x = pt_tri<false, false, BC>(x, Ads, Cfg::LDC, Ks, Cfg::LDQ, i0, j0, lane, tile_rows_lo<BC, DK>(it),
                                   tile_rows_hi<BC, DK>(it));
      if (ok) st4l(Zs, Cfg::LDQ, i0 + nn, j0 + 4 * gq, x);
    });
    __syncthreads();
    // W = L o D2 o (Q Z^T) (rows s, columns tau <= s);  Ek = L o D1 o (Zb K^T)
    for_causal_tiles<BC>(w, [&](int i0, int j0, bool ok, bool live) {
      f32x4 x = zero4();
      if (live) x = pt<false, true, DK>(x, Qs, Cfg::LDQ, Zs, Cfg::LDQ, i0, j0, lane);
      const int s = i0 + nn;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tau = j0 + 4 * gq + e;
        // the factor is read and applied on every lane (clamped index, masked value) so
        // that no branch forms around the table read
        x[e] = (tau <= s ? x[e] : 0.f) * pw[tau <= s ? 2 * (s - tau) : 0];
      }
      if (ok) st4l(Ws, Cfg::LDC, s, j0 + 4 * gq, x);
    });
    for_causal_tiles<BC>(w, [&](int i0, int j0, bool ok, bool live) {
      f32x4 x = zero4();
      if (live) x = pt<false, true, DK>(x, Zbs, Cfg::LDQ, Ks, Cfg::LDQ, i0, j0, lane);
      const int tr = i0 + nn;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ti = j0 + 4 * gq + e;
        // the factor is read and applied on every lane (clamped index, masked value) so
        // that no branch forms around the table read
        x[e] = (ti <= tr ? x[e] : 0.f) * pw[ti <= tr ? tr - ti : 0];
      }
      if (ok) st4l(Eks, Cfg::LDC, tr, j0 + 4 * gq, x);
    });
    __syncthreads();
    // dV' = W^T G' + diag(g^(2(BC-tau))) Z Ubar
    for_tiles<BC, DVP>(w, [&](int i0, int j0, bool ok, int it) {
      f32x4 x = pt<false, false, DK>(zero4(), Zs, Cfg::LDQ, Ubs, Cfg::LDV, i0, j0, lane);
      x *= pw[2 * (BC - (i0 + nn))];
      x = pt_tri<true, false, BC>(x, Ws, Cfg::LDC, Gs, Cfg::LDV, i0, j0, lane, tile_rows_lo<BC, DVP>(it),
                                  tile_rows_hi<BC, DVP>(it));
      if (ok) st_out(dvh, a.dv, t0 + i0 + nn, j0 + 4 * gq, a.n, x);
    });
    // dQ = diag(g^(tau+1)) [diag(g^(tau+1)) G' U0'^T + Zb S0] + Bm Z + Ek K
    for_tiles<BC, DK>(w, [&](int i0, int j0, bool ok, int it) {
      const int rlo = tile_rows_lo<BC, DK>(it), rhi = tile_rows_hi<BC, DK>(it);
      const float gt = pw[i0 + nn + 1];
      f32x4 x = pt_frags<DVP>(zero4(), u0f, Gs, Cfg::LDV, i0, lane);
      x *= gt;
      x = pt_frags<DK>(x, s0f, Zbs, Cfg::LDQ, i0, lane);
      x *= gt;
      x = pt_tri<false, false, BC>(x, Bms, Cfg::LDC, Zs, Cfg::LDQ, i0, j0, lane, rlo, rhi);
      x = pt_tri<false, false, BC>(x, Eks, Cfg::LDC, Ks, Cfg::LDQ, i0, j0, lane, rlo, rhi);
      if (ok) st_out(dqh, a.d, t0 + i0 + nn, j0 + 4 * gq, a.n, x);
    });
    // dK = Ad^T Zb + Ek^T Q + diag(g^(BC-tau)) K Shat
    for_tiles<BC, DK>(w, [&](int i0, int j0, bool ok, int it) {
      const int rlo = tile_rows_lo<BC, DK>(it), rhi = tile_rows_hi<BC, DK>(it);
      f32x4 x = pt<false, true, DK>(zero4(), Ks, Cfg::LDQ, Shs, Cfg::LDQ, i0, j0, lane);
      x *= pw[BC - (i0 + nn)];
      x = pt_tri<true, false, BC>(x, Ads, Cfg::LDC, Zbs, Cfg::LDQ, i0, j0, lane, rlo, rhi);
      x = pt_tri<true, false, BC>(x, Eks, Cfg::LDC, Qs, Cfg::LDQ, i0, j0, lane, rlo, rhi);
      if (ok) st_out(dkh, a.d, t0 + i0 + nn, j0 + 4 * gq, a.n, x);
    });
    bwd_adjoint_update<T, DK, DVP, BC, NW, Cfg, Cfg::QT>(smem, pw, w, lane, Ub, Sh);
    __syncthreads();  // every read of this chunk's LDS done
    bwd_adjoint_copy<T, DK, DVP, NW, true, Cfg>(smem, w, lane, Ub, Sh);
  }
}

}  // namespace hla2
