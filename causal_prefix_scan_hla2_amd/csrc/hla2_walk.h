// hla2_walk.h -- the chunk walker: one workgroup walks the chunks of one
// segment of one (b, h) sequence, carrying the corrected second-order state
// in registers.
//
// Method (technical summary of arXiv 2510.27258 on gist.science, §1 and §4).
// Per token t, with q_t, k_t in R^d, v_t in R^dv and decay g:
//   S_t = g S_{t-1} + k_t k_t^T                    (key moment)
//   z_t = S_t q_t
//   U_t = g^2 U_{t-1} + z_t v_t^T,  u_t = g^2 u_{t-1} + z_t
//   num_t = q_t^T U_t,  den_t = q_t^T u_t.
// U_t is the corrected product S_t C_t - G_t of the summary's output formula
// written as one state (U_t = sum_{i<=j<=t} g^{(t-i)+(t-j)} k_i (k_i.q_j) v_j^T),
// and u_t = S_t m_t - h_t is the matching denominator state.
//
// Chunk form.  For a chunk of `len` tokens (local index tau) entering with
// state (S0, U0, u0):
//   A   = Q K^T (chunk-local),  Ad[tau][i] = [i <= tau] g^{tau-i} A[tau][i]
//   Z   = diag(g^{tau+1}) Q S0 + Ad K                 (rows z_tau = S_tau q_tau)
//   W   = [j <= tau] g^{2(tau-j)} (Q Z^T)[tau][j]
//   num = diag(g^{2(tau+1)}) Q U0 + W V,  den = diag(g^{2(tau+1)}) Q u0 + W 1
//   S  <- g^len S0 + sum_t g^{len-1-t} k_t k_t^T
//   U  <- g^{2 len} U0 + sum_t g^{2(len-1-t)} z_t v_t^T,  u likewise with 1
// and, for segment summaries, C <- g^len C + sum_t g^{len-1-t} q_t v_t^T,
// m <- g^len m + sum_t g^{len-1-t} q_t.
//
// Work split inside the workgroup (4 waves).  The chunk's 16-row blocks of
// tokens are owned by waves: a wave computes A, Z, W and the outputs of its own
// rows, keeping Q, the masked A block and W as MFMA operand fragments in
// registers.  K, V, Z (transposed), S0 (bf16 copy) and U0^T (bf16 copy) live in
// LDS; K and Z share one buffer.  The fp32 states S, U (and C) stay in
// accumulator registers, split across the waves by 16-row blocks.
#pragma once
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

template <typename T, int DK, int DV, int CP, bool OUT>
struct WalkCfg {
  static constexpr int NW = 4;                       // waves per workgroup
  static constexpr int KR = Ktile<T>::ROWS;          // k-values per k-tile
  static constexpr int PADE = 16 / (int)sizeof(T);   // 16-byte row padding
  static constexpr int E = 16 / (int)sizeof(T);      // elements per 16-byte vector
  static constexpr int LDK = DK + PADE;              // K, Q, S0^T, U0^T rows
  static constexpr int LDV = DV + PADE;              // V rows
  static constexpr int LDZ = CP + PADE;              // Z^T rows
  static constexpr int NB = CP / 16;                 // 16-row token blocks
  static constexpr int TPW = (NB + NW - 1) / NW;     // token blocks per wave
  static constexpr int NKD = DK / KR;                // k-tiles over d
  static constexpr int NKC = CP / KR;                // k-tiles over chunk tokens
  static constexpr int RBS = DK / 16;                // 16-row blocks of S, U, C
  static constexpr int RPW = (RBS + NW - 1) / NW;    // state row blocks per wave
  static constexpr int CBS = DK / 16;
  static constexpr int CBU = DV / 16;
  static constexpr int KZ_ELEMS = (CP * LDK > DK * LDZ) ? CP * LDK : DK * LDZ;
  static constexpr int V_ELEMS = CP * LDV;
  static constexpr int X_ELEMS = DK * LDK;
  static constexpr int U_ELEMS = OUT ? DV * LDK : 0;
  static constexpr int Q_ELEMS = OUT ? 0 : CP * LDK;
  static constexpr int LDS_ELEMS = KZ_ELEMS + V_ELEMS + X_ELEMS + U_ELEMS + Q_ELEMS;
  static constexpr int LDS_BYTES = LDS_ELEMS * (int)sizeof(T) + 2 * DK * 4;
  static constexpr int NLK = (CP * DK / E + 255) / 256;  // 16-byte loads per thread, K (and Q)
  static constexpr int NLV = (CP * DV / E + 255) / 256;  // 16-byte loads per thread, V
  static constexpr int WAVES_PER_EU = (LDS_BYTES <= 80 * 1024) ? 2 : 1;
  static_assert(DK % KR == 0 && CP % KR == 0, "tile sizes must be multiples of the k-tile");
  static_assert(DK % 16 == 0 && DV % 16 == 0 && CP % 16 == 0, "16-multiples");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// token-block index owned by wave w in its slot tb (pairs early and late blocks
// when a wave owns two, so every wave gets a similar share of the causal work)
template <int NB, int NW, int TPW>
__device__ __forceinline__ int tau_block(int w, int tb) {
  if (TPW == 2 && NB == 2 * NW) return tb == 0 ? w : NB - 1 - w;
  return w + tb * NW;
}

template <typename T, int DK, int DV, int CP, bool OUT>
__global__ void __launch_bounds__(256, (WalkCfg<T, DK, DV, CP, OUT>::WAVES_PER_EU))
walk_kernel(WalkArgs a) {
  using Cfg = WalkCfg<T, DK, DV, CP, OUT>;
  using frag = typename Ktile<T>::frag;
  constexpr int NW = Cfg::NW, KR = Cfg::KR, E = Cfg::E;
  constexpr int LDK = Cfg::LDK, LDV = Cfg::LDV, LDZ = Cfg::LDZ;
  constexpr int NB = Cfg::NB, TPW = Cfg::TPW, NKD = Cfg::NKD, NKC = Cfg::NKC;
  constexpr int RBS = Cfg::RBS, RPW = Cfg::RPW, CBS = Cfg::CBS, CBU = Cfg::CBU;
  constexpr int NLK = Cfg::NLK, NLV = Cfg::NLV;
  constexpr bool BF = sizeof(T) == 2;

  __shared__ __attribute__((aligned(16))) T smem[Cfg::LDS_ELEMS];
  __shared__ float u0s[DK];
  T *KZ = smem;                          // K rows [CP][LDK]  /  Z^T rows [DK][LDZ]
  T *Vs = KZ + Cfg::KZ_ELEMS;            // V rows [CP][LDV]
  T *X = Vs + Cfg::V_ELEMS;              // S0^T rows [DK][LDK] (bf16/f32 copy of the state)
  T *U0t = X + Cfg::X_ELEMS;             // U0^T rows [DV][LDK] (output mode)
  T *Qs = U0t + Cfg::U_ELEMS;            // Q rows [CP][LDK]    (summary mode)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, nl = lane & 15;
  const int nseg_here = OUT ? a.nseg : a.nseg - 1;
  const int bh = blockIdx.x / nseg_here, seg = blockIdx.x % nseg_here;
  const long tok0 = (long)seg * a.cps * a.chunk;
  const long tokE = ((long)a.n < tok0 + (long)a.cps * a.chunk) ? (long)a.n : tok0 + (long)a.cps * a.chunk;
  const int nch = (int)((tokE - tok0 + a.chunk - 1) / a.chunk);
  const T *qg = (const T *)a.q + (long)bh * a.n * a.d;
  const T *kg = (const T *)a.k + (long)bh * a.n * a.d;
  const T *vg = (const T *)a.v + (long)bh * a.n * a.dv;
  const float log2g = a.log2g;
  const bool dec = a.decay_on != 0;
  auto gp = [&](float x) __attribute__((always_inline)) -> float { return dec ? exp2f(x * log2g) : 1.0f; };

  // ---------------- state registers ----------------
  f32x4 Sacc[RPW][CBS], Uacc[RPW][CBU], Cacc[OUT ? 1 : RPW][OUT ? 1 : CBU];
  float ureg = 0.f, mreg = 0.f;  // thread tid < DK keeps u[tid] (and m[tid] in summary mode)
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
#pragma unroll
    for (int cb = 0; cb < CBS; ++cb) Sacc[i][cb] = zero4();
#pragma unroll
    for (int cb = 0; cb < CBU; ++cb) Uacc[i][cb] = zero4();
  }
  if constexpr (!OUT) {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int cb = 0; cb < CBU; ++cb) Cacc[i][cb] = zero4();
  }
  if (OUT && seg > 0) {
    const float *pb = a.prefix + ((long)bh * a.nseg + seg) * prefix_block_floats(DK, DV);
    const float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = w + i * NW;
      if (rb < RBS) {
#pragma unroll
        for (int cb = 0; cb < CBS; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) Sacc[i][cb][r] = pS[(16 * rb + 4 * g + r) * DK + 16 * cb + nl];
#pragma unroll
        for (int cb = 0; cb < CBU; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) Uacc[i][cb][r] = pU[(16 * rb + 4 * g + r) * DV + 16 * cb + nl];
      }
    }
    if (tid < DK) ureg = pu[tid];
  }

  // copy the state into LDS as MFMA operands: S0^T rows and U0^T rows
  auto write_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = w + i * NW;
      if (rb < RBS) {
#pragma unroll
        for (int cb = 0; cb < CBS; ++cb) st4(X + (16 * cb + nl) * LDK + 16 * rb + 4 * g, Sacc[i][cb]);
        if constexpr (OUT) {
#pragma unroll
          for (int cb = 0; cb < CBU; ++cb) st4(U0t + (16 * cb + nl) * LDK + 16 * rb + 4 * g, Uacc[i][cb]);
        }
      }
    }
    if (OUT && tid < DK) u0s[tid] = ureg;
  };

  // ---------------- chunk staging ----------------
  uint4 kreg[NLK], vreg[NLV], qreg[OUT ? 1 : NLK];
  frag qf[TPW][NKD], qn[OUT ? TPW : 1][OUT ? NKD : 1];

  auto chunk_len = [&](int c) __attribute__((always_inline)) -> int {
    const long t0 = tok0 + (long)c * a.chunk;
    const long r = tokE - t0;
    return r < a.chunk ? (int)r : a.chunk;
  };
  auto load_regs = [&](int c) __attribute__((always_inline)) {
    const long t0 = tok0 + (long)c * a.chunk;
    const int len = chunk_len(c);
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = (i * 256 + tid) * E;
      const int t = e / DK, col = e % DK;
      const bool ok = e < CP * DK && t < len && col < a.d;
      const long off = ok ? (t0 + t) * a.d + col : 0;
      kreg[i] = ld_or_zero((const uint4 *)(kg + off), (const uint4 *)kg, ok);
      if constexpr (!OUT) qreg[i] = ld_or_zero((const uint4 *)(qg + off), (const uint4 *)qg, ok);
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = (i * 256 + tid) * E;
      const int t = e / DV, col = e % DV;
      const bool ok = e < CP * DV && t < len && col < a.dv;
      const long off = ok ? (t0 + t) * a.dv + col : 0;
      vreg[i] = ld_or_zero((const uint4 *)(vg + off), (const uint4 *)vg, ok);
    }
  };
  auto store_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = (i * 256 + tid) * E;
      if (e < CP * DK) {
        *(uint4 *)(KZ + (e / DK) * LDK + e % DK) = kreg[i];
        if constexpr (!OUT) *(uint4 *)(Qs + (e / DK) * LDK + e % DK) = qreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = (i * 256 + tid) * E;
      if (e < CP * DV) *(uint4 *)(Vs + (e / DV) * LDV + e % DV) = vreg[i];
    }
  };
  // Q operand fragments of the wave's own token rows, straight from global memory
  auto load_q = [&](int c, frag (&dst)[OUT ? TPW : 1][OUT ? NKD : 1]) __attribute__((always_inline)) {
    if constexpr (OUT) {
      const long t0 = tok0 + (long)c * a.chunk;
      const int len = chunk_len(c);
#pragma unroll
      for (int tb = 0; tb < TPW; ++tb) {
        const int Tb = tau_block<NB, NW, TPW>(w, tb);
        const int tau = 16 * Tb + nl;
        const bool rowok = Tb < NB && tau < len;
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
          if constexpr (BF) {
            const int c0 = kd * KR + 4 * g, c1 = c0 + 16;
            const T *row = qg + (rowok ? (t0 + tau) * a.d : 0);
            bf16x4 lo = ld_or_zero((const bf16x4 *)(row + c0), (const bf16x4 *)qg, rowok && c0 < a.d);
            bf16x4 hi = ld_or_zero((const bf16x4 *)(row + c1), (const bf16x4 *)qg, rowok && c1 < a.d);
            dst[tb][kd] = cat8(lo, hi);
          } else {
            const int c0 = kd * KR + 4 * g;
            const T *row = qg + (rowok ? (t0 + tau) * a.d : 0);
            dst[tb][kd] = ld_or_zero((const f32x4 *)(row + c0), (const f32x4 *)qg, rowok && c0 < a.d);
          }
        }
      }
    }
  };

  // ---------------- prologue ----------------
  if (nch > 0) {
    load_regs(0);
    if constexpr (OUT) load_q(0, qn);
  }
  write_state();
  if (nch > 0) store_lds();
  if constexpr (OUT) {
#pragma unroll
    for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) qf[tb][kd] = qn[tb][kd];
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const long t0 = tok0 + (long)c * a.chunk;
    const int len = chunk_len(c);
    const float Gam = gp((float)len);
    if (c + 1 < nch) {
      load_regs(c + 1);
      if constexpr (OUT) load_q(c + 1, qn);
    }
    if constexpr (!OUT) {
#pragma unroll
      for (int tb = 0; tb < TPW; ++tb) {
        const int Tb = tau_block<NB, NW, TPW>(w, tb);
        if (Tb < NB) {
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) qf[tb][kd] = ld_rows(Qs, LDK, 16 * Tb, kd * KR, lane);
        }
      }
    }

    // ---- A^T = K Q^T for the wave's rows, masked and decayed -> operand fragments of Ad
    frag adf[TPW][NKC];
    f32x4 zacc[TPW][CBS];
#pragma unroll
    for (int tb = 0; tb < TPW; ++tb) {
      const int Tb = tau_block<NB, NW, TPW>(w, tb);
      if (Tb < NB) {
        f32x4 at[NB];
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          at[I] = zero4();
          if (I <= Tb) {
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) at[I] = mma(ld_rows(KZ, LDK, 16 * I, kd * KR, lane), qf[tb][kd], at[I]);
            const int tau = 16 * Tb + nl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 16 * I + 4 * g + r;
              at[I][r] = (i <= tau) ? at[I][r] * gp((float)(tau - i)) : 0.f;
            }
          }
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          if constexpr (BF) adf[tb][kc] = frag_from_acc(at[2 * kc], at[2 * kc + 1]);
          else adf[tb][kc] = frag_from_acc(at[kc]);
        }
        // ---- Z = diag(g^{tau+1}) Q S0 + Ad K
#pragma unroll
        for (int acb = 0; acb < CBS; ++acb) {
          f32x4 z = zero4();
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) z = mma(qf[tb][kd], ld_rows(X, LDK, 16 * acb, kd * KR, lane), z);
#pragma unroll
          for (int r = 0; r < 4; ++r) z[r] *= gp((float)(16 * Tb + 4 * g + r + 1));
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc)
            if (kc * KR <= 16 * Tb + 15) z = mma(adf[tb][kc], ld_cols(KZ, LDK, kc * KR, 16 * acb, lane), z);
          zacc[tb][acb] = z;
        }
      }
    }

    // ---- S <- g^len S + sum_t g^{len-1-t} k_t k_t^T   (and C in summary mode, later)
    {
      auto wk = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? gp((float)(len - 1 - t)) : 0.f;
        };
      };
#pragma unroll
      for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int cb = 0; cb < CBS; ++cb) Sacc[i][cb] *= Gam;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        frag af[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int rb = w + i * NW;
          if (rb < RBS) af[i] = scale_frag(ld_cols(KZ, LDK, kc * KR, 16 * rb, lane), g, wk(kc * KR));
        }
#pragma unroll
        for (int cb = 0; cb < CBS; ++cb) {
          frag b = ld_cols(KZ, LDK, kc * KR, 16 * cb, lane);
#pragma unroll
          for (int i = 0; i < RPW; ++i)
            if (w + i * NW < RBS) Sacc[i][cb] = mma(af[i], b, Sacc[i][cb]);
        }
      }
    }
    __syncthreads();  // every read of K and S0 is done

    // ---- Z^T into the K/Z buffer
#pragma unroll
    for (int tb = 0; tb < TPW; ++tb) {
      const int Tb = tau_block<NB, NW, TPW>(w, tb);
      if (Tb < NB) {
#pragma unroll
        for (int acb = 0; acb < CBS; ++acb) st4(KZ + (16 * acb + nl) * LDZ + 16 * Tb + 4 * g, zacc[tb][acb]);
      }
    }
    __syncthreads();

    // ---- denominator state and query mass (plain sums over the chunk)
    float unext = ureg;
    if (tid < DK) {
      const float G2 = Gam * Gam;
      float su = 0.f;
      for (int t = 0; t < len; ++t) su += gp(2.f * (float)(len - 1 - t)) * (float)KZ[tid * LDZ + t];
      unext = G2 * ureg + su;
      if constexpr (!OUT) {
        float sm = 0.f;
        for (int t = 0; t < len; ++t) sm += gp((float)(len - 1 - t)) * (float)Qs[t * LDK + tid];
        mreg = Gam * mreg + sm;
      }
    }

    if constexpr (OUT) {
      // ---- W^T = Z Q^T (masked, decayed) -> operand fragments; den; outputs
#pragma unroll
      for (int tb = 0; tb < TPW; ++tb) {
        const int Tb = tau_block<NB, NW, TPW>(w, tb);
        if (Tb < NB) {
          const int tau = 16 * Tb + nl;
          f32x4 wt[NB];
          float rs = 0.f;
#pragma unroll
          for (int J = 0; J < NB; ++J) {
            wt[J] = zero4();
            if (J <= Tb) {
#pragma unroll
              for (int kd = 0; kd < NKD; ++kd) wt[J] = mma(ld_cols(KZ, LDZ, kd * KR, 16 * J, lane), qf[tb][kd], wt[J]);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int j = 16 * J + 4 * g + r;
                wt[J][r] = (j <= tau) ? wt[J][r] * gp(2.f * (float)(tau - j)) : 0.f;
                rs += wt[J][r];
              }
            }
          }
          frag wf[NKC];
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            if constexpr (BF) wf[kc] = frag_from_acc(wt[2 * kc], wt[2 * kc + 1]);
            else wf[kc] = frag_from_acc(wt[kc]);
          }
          // q_tau . u0 from the wave's Q fragments
          float qu = 0.f;
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) {
#pragma unroll
            for (int e = 0; e < (BF ? 8 : 4); ++e) qu += (float)qf[tb][kd][e] * u0s[kd * KR + kidx<T>(g, e)];
          }
          const float carry2 = gp(2.f * (float)(tau + 1));
          const float den = carry2 * sum_groups(qu) + sum_groups(rs);
          const bool rowok = tau < len;
          if (a.den_out && g == 0 && rowok) a.den_out[(long)bh * a.n + t0 + tau] = den;
          T *orow = (T *)a.out + ((long)bh * a.n + t0 + tau) * a.dv;
#pragma unroll
          for (int cb = 0; cb < CBU; ++cb) {
            f32x4 o = zero4();
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) o = mma(ld_rows(U0t, LDK, 16 * cb, kd * KR, lane), qf[tb][kd], o);
            o *= carry2;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
              if (kc * KR <= 16 * Tb + 15) o = mma(ld_cols(Vs, LDV, kc * KR, 16 * cb, lane), wf[kc], o);
            if (a.normalize) {
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = o[r] / den;
            }
            if (rowok && 16 * cb < a.dv) st4(orow + 16 * cb + 4 * g, o);
          }
        }
      }
    }

    // ---- U <- g^{2len} U + sum_t g^{2(len-1-t)} z_t v_t^T ;  C likewise with q (summary)
    {
      const float G2 = Gam * Gam;
      auto wz = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? gp(2.f * (float)(len - 1 - t)) : 0.f;
        };
      };
      auto wq = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? gp((float)(len - 1 - t)) : 0.f;
        };
      };
#pragma unroll
      for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int cb = 0; cb < CBU; ++cb) {
          Uacc[i][cb] *= G2;
          if constexpr (!OUT) Cacc[i][cb] *= Gam;
        }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        frag af[RPW], aq[OUT ? 1 : RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int rb = w + i * NW;
          if (rb < RBS) {
            af[i] = scale_frag(ld_rows(KZ, LDZ, 16 * rb, kc * KR, lane), g, wz(kc * KR));
            if constexpr (!OUT) aq[i] = scale_frag(ld_cols(Qs, LDK, kc * KR, 16 * rb, lane), g, wq(kc * KR));
          }
        }
#pragma unroll
        for (int cb = 0; cb < CBU; ++cb) {
          frag b = ld_cols(Vs, LDV, kc * KR, 16 * cb, lane);
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            if (w + i * NW < RBS) {
              Uacc[i][cb] = mma(af[i], b, Uacc[i][cb]);
              if constexpr (!OUT) Cacc[i][cb] = mma(aq[i], b, Cacc[i][cb]);
            }
          }
        }
      }
    }
    __syncthreads();  // every read of Z, V, S0, U0 and u0 is done
    ureg = unext;
    write_state();
    if (c + 1 < nch) {
      store_lds();
      if constexpr (OUT) {
#pragma unroll
        for (int tb = 0; tb < TPW; ++tb)
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) qf[tb][kd] = qn[tb][kd];
      }
    }
    __syncthreads();
  }

  if constexpr (!OUT) {
    // segment summary: S | C | U | m | u
    float *sb = a.sums + ((long)bh * (a.nseg - 1) + seg) * sum_block_floats(DK, DV);
    float *sS = sb, *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = w + i * NW;
      if (rb < RBS) {
#pragma unroll
        for (int cb = 0; cb < CBS; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) sS[(16 * rb + 4 * g + r) * DK + 16 * cb + nl] = Sacc[i][cb][r];
#pragma unroll
        for (int cb = 0; cb < CBU; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sC[(16 * rb + 4 * g + r) * DV + 16 * cb + nl] = Cacc[i][cb][r];
            sU[(16 * rb + 4 * g + r) * DV + 16 * cb + nl] = Uacc[i][cb][r];
          }
      }
    }
    if (tid < DK) {
      sm[tid] = mreg;
      su[tid] = ureg;
    }
  }
}

// Instantiate and launch one (T, DK, DV, CP) pair of walker kernels.
template <typename T, int DK, int DV, int CP>
hipError_t launch_walk_t(bool output_mode, dim3 grid, const WalkArgs &a, hipStream_t s) {
  if (output_mode)
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, CP, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, CP, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hla2
