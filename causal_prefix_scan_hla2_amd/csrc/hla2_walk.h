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
// Work split inside the workgroup.  Every wave owns one 16-row block of the
// chunk's tokens and computes A, Z, W and the outputs of its rows, keeping Q,
// the masked A block and W as MFMA operand fragments in registers.  K, V,
// Z (as Z^T), S0 and U0^T (bf16 copies of the state) live in LDS; K and Z share
// one buffer.  The fp32 states S, U, u (and C, m) stay in accumulator
// registers, split across the waves by 16x16 tiles.  Sums over the chunk's
// tokens (u, m) ride along the state products as one extra all-ones column.
#pragma once
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

template <typename T, int DK, int DV, int CP, bool OUT>
struct WalkCfg {
  static constexpr int NB = CP / 16;                 // 16-row token blocks
  static constexpr int NW = NB > 4 ? NB : 4;         // waves per workgroup
  static constexpr int NT = 64 * NW;                 // threads
  static constexpr int KR = Ktile<T>::ROWS;          // k-values per k-tile
  static constexpr int PADE = 16 / (int)sizeof(T);   // 16-byte row padding
  static constexpr int E = 16 / (int)sizeof(T);      // elements per 16-byte vector
  static constexpr int LDK = DK + PADE;              // K, Q, S0^T, U0^T rows
  static constexpr int LDV = DV + PADE;              // V rows
  static constexpr int LDZ = CP + PADE;              // Z^T rows
  static constexpr int NKD = DK / KR;                // k-tiles over d
  static constexpr int NKC = CP / KR;                // k-tiles over chunk tokens
  static constexpr int RBS = DK / 16;                // 16-row blocks of S, U, C
  static constexpr int CBS = DK / 16;
  static constexpr int CBU = DV / 16;
  // state tiles: waves split the row blocks, and the column blocks too when
  // there are fewer row blocks than waves
  static constexpr bool ROWSPLIT = RBS >= NW;
  static constexpr int RPW = ROWSPLIT ? RBS / NW : 1;
  static constexpr int CSN = ROWSPLIT ? 1 : NW / RBS;
  static constexpr int CPW_S = (CBS + CSN - 1) / CSN;
  static constexpr int CPW_U = (CBU + CSN - 1) / CSN;
  static constexpr int KZ_ELEMS = (CP * LDK > DK * LDZ) ? CP * LDK : DK * LDZ;
  static constexpr int V_ELEMS = CP * LDV;
  static constexpr int X_ELEMS = DK * LDK;
  static constexpr int U_ELEMS = OUT ? DV * LDK : 0;
  static constexpr int Q_ELEMS = OUT ? 0 : CP * LDK;
  static constexpr int LDS_ELEMS = KZ_ELEMS + V_ELEMS + X_ELEMS + U_ELEMS + Q_ELEMS;
  static constexpr int LDS_BYTES = walk_lds_bytes((int)sizeof(T), DK, DV, CP, OUT);
  static constexpr int NLK = (CP * DK / E + NT - 1) / NT;  // 16-byte loads per thread, K (and Q)
  static constexpr int NLV = (CP * DV / E + NT - 1) / NT;  // 16-byte loads per thread, V
  static constexpr int WAVES_PER_EU = walk_waves_per_eu((int)sizeof(T), DK, DV, CP, OUT);
  static_assert(LDS_ELEMS * (int)sizeof(T) + (2 * CP + 1 + DK) * 4 <= LDS_BYTES, "LDS accounting");
  static_assert(DK % KR == 0 && CP % KR == 0, "tile sizes must be multiples of the k-tile");
  static_assert(DK % 16 == 0 && DV % 16 == 0 && CP % 16 == 0, "16-multiples");
  static_assert(ROWSPLIT ? RBS % NW == 0 : NW % RBS == 0, "state tile split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// 16-row token block owned by wave w.  With eight blocks, waves w and w+4 (which
// share a SIMD) get blocks whose causal work adds up to the same amount.
template <int NB>
__device__ __forceinline__ int tau_block(int w) {
  if (NB == 8) return w < 4 ? w : 11 - w;
  return w;
}

template <typename T, int DK, int DV, int CP, bool OUT>
__global__ void __launch_bounds__((WalkCfg<T, DK, DV, CP, OUT>::NT), (WalkCfg<T, DK, DV, CP, OUT>::WAVES_PER_EU))
walk_kernel(WalkArgs a) {
  using Cfg = WalkCfg<T, DK, DV, CP, OUT>;
  using frag = typename Ktile<T>::frag;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, KR = Cfg::KR, E = Cfg::E;
  constexpr int LDK = Cfg::LDK, LDV = Cfg::LDV, LDZ = Cfg::LDZ;
  constexpr int NB = Cfg::NB, NKD = Cfg::NKD, NKC = Cfg::NKC;
  constexpr int RBS = Cfg::RBS, RPW = Cfg::RPW, CSN = Cfg::CSN, CBS = Cfg::CBS, CBU = Cfg::CBU;
  constexpr int CPW_S = Cfg::CPW_S, CPW_U = Cfg::CPW_U;
  constexpr bool ROWSPLIT = Cfg::ROWSPLIT;
  constexpr int NLK = Cfg::NLK, NLV = Cfg::NLV;
  constexpr bool BF = sizeof(T) == 2;

  __shared__ __attribute__((aligned(16))) T smem[Cfg::LDS_ELEMS];
  __shared__ float pw[2 * CP + 1];  // decay^x, x = 0 .. 2 CP
  __shared__ float u0s[DK];         // u0 (fp32) for the denominator's carried term
  T *KZ = smem;                     // K rows [CP][LDK]  /  Z^T rows [DK][LDZ]
  T *Vs = KZ + Cfg::KZ_ELEMS;       // V rows [CP][LDV]
  T *X = Vs + Cfg::V_ELEMS;         // S0^T rows [DK][LDK]
  T *U0t = X + Cfg::X_ELEMS;        // U0^T rows [DV][LDK] (output mode)
  T *Qs = U0t + Cfg::U_ELEMS;       // Q rows [CP][LDK]    (summary mode)

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, nl = lane & 15;
  // the wave index is uniform across the wave: keep it in a scalar register so that every
  // branch on it (token block, state tiles) is a scalar branch around whole-wave MFMA code
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nseg_here = OUT ? a.nseg : walk_nsum(a);
  const int bh = blockIdx.x / nseg_here, seg = blockIdx.x % nseg_here;
  const long tok0 = (long)seg * a.cps * a.chunk;
  const long tokE = ((long)a.n < tok0 + (long)a.cps * a.chunk) ? (long)a.n : tok0 + (long)a.cps * a.chunk;
  // a summary of the last segment (final state) stops at its last full chunk
  const int nch = (!OUT && seg == a.nseg - 1) ? (int)((tokE - tok0) / a.chunk)
                                              : (int)((tokE - tok0 + a.chunk - 1) / a.chunk);
  const T *qg = (const T *)a.q + (long)bh * a.n * a.d;
  const T *kg = (const T *)a.k + (long)bh * a.n * a.d;
  const T *vg = (const T *)a.v + (long)bh * a.n * a.dv;
  const bool dec = a.decay_on != 0;
  const bool need_den = a.need_den != 0;
  auto P = [&](int x) __attribute__((always_inline)) -> float { return dec ? pw[x] : 1.0f; };
  for (int x = tid; x <= 2 * CP; x += NT) pw[x] = dec ? exp2f((float)x * a.log2g) : 1.0f;

  // state tile ownership of this wave
  auto srow = [&](int i) __attribute__((always_inline)) -> int { return ROWSPLIT ? w + i * NW : w % RBS; };
  auto scol = [&](int j) __attribute__((always_inline)) -> int { return ROWSPLIT ? j : w / RBS + j * CSN; };
  const bool ones_owner = ROWSPLIT || (w / RBS) == 0;  // waves that carry the all-ones column (u, m)

  // ---------------- state registers ----------------
  f32x4 Sacc[RPW][CPW_S], Uacc[RPW][CPW_U], Cacc[OUT ? 1 : RPW][OUT ? 1 : CPW_U];
  f32x4 uacc[RPW], macc[OUT ? 1 : RPW];  // column 0 of the all-ones products: u (and m)
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
#pragma unroll
    for (int j = 0; j < CPW_S; ++j) Sacc[i][j] = zero4();
#pragma unroll
    for (int j = 0; j < CPW_U; ++j) Uacc[i][j] = zero4();
    uacc[i] = zero4();
    if constexpr (!OUT) {
      macc[i] = zero4();
#pragma unroll
      for (int j = 0; j < CPW_U; ++j) Cacc[i][j] = zero4();
    }
  }
  if (OUT && seg > 0) {
    const float *pb = a.prefix + ((long)bh * a.nseg + seg) * prefix_block_floats(DK, DV);
    const float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = srow(i);
#pragma unroll
      for (int j = 0; j < CPW_S; ++j) {
        const int cb = scol(j);
        if (cb < CBS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Sacc[i][j][r] = pS[(16 * rb + 4 * g + r) * DK + 16 * cb + nl];
        }
      }
#pragma unroll
      for (int j = 0; j < CPW_U; ++j) {
        const int cb = scol(j);
        if (cb < CBU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Uacc[i][j][r] = pU[(16 * rb + 4 * g + r) * DV + 16 * cb + nl];
        }
      }
      if (ones_owner && nl == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) uacc[i][r] = pu[16 * rb + 4 * g + r];
      }
    }
  }

  // copy the state into LDS as MFMA operands: S0^T rows, U0^T rows and u0
  auto write_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = srow(i);
#pragma unroll
      for (int j = 0; j < CPW_S; ++j) {
        const int cb = scol(j);
        if (cb < CBS) st4(X + (16 * cb + nl) * LDK + 16 * rb + 4 * g, Sacc[i][j]);
      }
      if constexpr (OUT) {
#pragma unroll
        for (int j = 0; j < CPW_U; ++j) {
          const int cb = scol(j);
          if (cb < CBU) st4(U0t + (16 * cb + nl) * LDK + 16 * rb + 4 * g, Uacc[i][j]);
        }
        if (ones_owner && nl == 0) *(f32x4 *)(u0s + 16 * rb + 4 * g) = uacc[i];
      }
    }
  };

  // ---------------- chunk staging ----------------
  uint4 kreg[NLK], vreg[NLV], qreg[OUT ? 1 : NLK];
  const int Tb = tau_block<NB>(w);  // this wave's token block (>= NB: none)
  const bool has_rows = Tb < NB;
  frag qf[NKD], qn[OUT ? NKD : 1];

  auto chunk_len = [&](int c) __attribute__((always_inline)) -> int {
    const long r = tokE - (tok0 + (long)c * a.chunk);
    return r < a.chunk ? (int)r : a.chunk;
  };
  auto load_regs = [&](int c) __attribute__((always_inline)) {
    const long t0 = tok0 + (long)c * a.chunk;
    const int len = chunk_len(c);
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = (i * NT + tid) * E;
      const int t = e / DK, col = e % DK;
      const bool ok = e < CP * DK && t < len && col < a.d;
      const long off = ok ? (t0 + t) * a.d + col : 0;
      kreg[i] = ld_or_zero((const uint4 *)(kg + off), (const uint4 *)kg, ok);
      if constexpr (!OUT) qreg[i] = ld_or_zero((const uint4 *)(qg + off), (const uint4 *)qg, ok);
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = (i * NT + tid) * E;
      const int t = e / DV, col = e % DV;
      const bool ok = e < CP * DV && t < len && col < a.dv;
      const long off = ok ? (t0 + t) * a.dv + col : 0;
      vreg[i] = ld_or_zero((const uint4 *)(vg + off), (const uint4 *)vg, ok);
    }
  };
  auto store_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLK; ++i) {
      const int e = (i * NT + tid) * E;
      if (e < CP * DK) {
        *(uint4 *)(KZ + (e / DK) * LDK + e % DK) = kreg[i];
        if constexpr (!OUT) *(uint4 *)(Qs + (e / DK) * LDK + e % DK) = qreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int e = (i * NT + tid) * E;
      if (e < CP * DV) *(uint4 *)(Vs + (e / DV) * LDV + e % DV) = vreg[i];
    }
  };
  // Q operand fragments of the wave's own token rows, straight from global memory
  auto load_q = [&](int c, frag (&dst)[OUT ? NKD : 1]) __attribute__((always_inline)) {
    if constexpr (OUT) {
      const long t0 = tok0 + (long)c * a.chunk;
      const int len = chunk_len(c);
      const int tau = 16 * Tb + nl;
      const bool rowok = has_rows && tau < len;
      const T *row = qg + (rowok ? (t0 + tau) * a.d : 0);
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        if constexpr (BF) {
          const int c0 = kd * KR + 4 * g, c1 = c0 + 16;
          bf16x4 lo = ld_or_zero((const bf16x4 *)(row + c0), (const bf16x4 *)qg, rowok && c0 < a.d);
          bf16x4 hi = ld_or_zero((const bf16x4 *)(row + c1), (const bf16x4 *)qg, rowok && c1 < a.d);
          dst[kd] = cat8(lo, hi);
        } else {
          const int c0 = kd * KR + 4 * g;
          dst[kd] = ld_or_zero((const f32x4 *)(row + c0), (const f32x4 *)qg, rowok && c0 < a.d);
        }
      }
    }
  };
  // the all-ones column as a B operand: 1 in column 0, 0 elsewhere
  frag ones;
  {
    const float o = nl == 0 ? 1.0f : 0.0f;
    if constexpr (BF) {
      const bf16 b = (bf16)o;
      ones = bf16x8{b, b, b, b, b, b, b, b};
    } else {
      ones = f32x4{o, o, o, o};
    }
  }

  // ---------------- prologue ----------------
  if (nch > 0) {
    load_regs(0);
    if constexpr (OUT) load_q(0, qn);
  }
  write_state();
  if (nch > 0) store_lds();
  if constexpr (OUT) {
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = qn[kd];
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const long t0 = tok0 + (long)c * a.chunk;
    const int len = chunk_len(c);
    const float Gam = P(len), G2 = P(2 * len);
    if constexpr (!OUT) {
      if (has_rows) {
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) qf[kd] = ld_rows(Qs, LDK, 16 * Tb, kd * KR, lane);
      }
    }

    // ---- S <- g^len S + sum_t g^{len-1-t} k_t k_t^T
    {
      auto wk = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? P(len - 1 - t) : 0.f;
        };
      };
#pragma unroll
      for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int j = 0; j < CPW_S; ++j) Sacc[i][j] *= Gam;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        frag af[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          af[i] = ld_cols(KZ, LDK, kc * KR, 16 * srow(i), lane);
          if (dec) af[i] = scale_frag(af[i], g, wk(kc * KR));
        }
#pragma unroll
        for (int j = 0; j < CPW_S; ++j) {
          const int cb = scol(j);
          if (cb < CBS) {
            frag b = ld_cols(KZ, LDK, kc * KR, 16 * cb, lane);
#pragma unroll
            for (int i = 0; i < RPW; ++i) Sacc[i][j] = mma(af[i], b, Sacc[i][j]);
          }
        }
      }
    }
    // ---- A^T = K Q^T for the wave's rows, masked and decayed -> operand fragments of Ad
    frag adf[NKC];
    f32x4 zacc[CBS];
    if (has_rows) {
      const int tau = 16 * Tb + nl;
      f32x4 at[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        at[I] = zero4();
        if (I <= Tb) {
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) at[I] = mma(ld_rows(KZ, LDK, 16 * I, kd * KR, lane), qf[kd], at[I]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * g + r;
            at[I][r] = (i <= tau) ? at[I][r] * P(tau - i) : 0.f;
          }
        }
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if constexpr (BF) adf[kc] = frag_from_acc(at[2 * kc], at[2 * kc + 1]);
        else adf[kc] = frag_from_acc(at[kc]);
      }
      // ---- Z = diag(g^{tau+1}) Q S0 + Ad K
#pragma unroll
      for (int acb = 0; acb < CBS; ++acb) {
        f32x4 z = zero4();
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) z = mma(qf[kd], ld_rows(X, LDK, 16 * acb, kd * KR, lane), z);
        if (dec) {
#pragma unroll
          for (int r = 0; r < 4; ++r) z[r] *= pw[16 * Tb + 4 * g + r + 1];
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          if (kc * KR <= 16 * Tb + 15) z = mma(adf[kc], ld_cols(KZ, LDK, kc * KR, 16 * acb, lane), z);
        zacc[acb] = z;
      }
    }

    __syncthreads();  // every read of K and S0 is done

    // ---- Z^T into the K/Z buffer
    if (has_rows) {
#pragma unroll
      for (int acb = 0; acb < CBS; ++acb) st4(KZ + (16 * acb + nl) * LDZ + 16 * Tb + 4 * g, zacc[acb]);
    }
    // prefetch the next chunk; it lands in LDS after this chunk's last barrier
    if (c + 1 < nch) {
      load_regs(c + 1);
      if constexpr (OUT) load_q(c + 1, qn);
    }
    __syncthreads();

    if constexpr (OUT) {
      // ---- W^T = Z Q^T (masked, decayed) -> operand fragments; den; outputs
      if (has_rows) {
        const int tau = 16 * Tb + nl;
        f32x4 wt[NB];
        float rs = 0.f;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          wt[J] = zero4();
          if (J <= Tb) {
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) wt[J] = mma(ld_cols(KZ, LDZ, kd * KR, 16 * J, lane), qf[kd], wt[J]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * J + 4 * g + r;
              wt[J][r] = (j <= tau) ? wt[J][r] * P(2 * (tau - j)) : 0.f;
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
        const float carry2 = P(2 * (tau + 1));
        float den = 1.f;
        if (need_den) {
          // q_tau . u0 from the wave's Q fragments
          float qu = 0.f;
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) {
#pragma unroll
            for (int e = 0; e < (BF ? 8 : 4); ++e) qu += (float)qf[kd][e] * u0s[kd * KR + kidx<T>(g, e)];
          }
          den = carry2 * sum_groups(qu) + sum_groups(rs);
        }
        const bool rowok = tau < len;
        if (a.den_out && g == 0 && rowok) a.den_out[(long)bh * a.n + t0 + tau] = den;
        T *orow = (T *)a.out + ((long)bh * a.n + t0 + (rowok ? tau : 0)) * a.dv;
#pragma unroll
        for (int cb = 0; cb < CBU; ++cb) {
          f32x4 o = zero4();
#pragma unroll
          for (int kd = 0; kd < NKD; ++kd) o = mma(ld_rows(U0t, LDK, 16 * cb, kd * KR, lane), qf[kd], o);
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

    // ---- U <- g^{2len} U + sum_t g^{2(len-1-t)} z_t v_t^T (u with the ones column);
    //      C, m likewise with q in summary mode
    {
      auto wz = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? P(2 * (len - 1 - t)) : 0.f;
        };
      };
      auto wq = [&](int kbase) __attribute__((always_inline)) {
        return [=](int kk) __attribute__((always_inline)) -> float {
          const int t = kbase + kk;
          return t < len ? P(len - 1 - t) : 0.f;
        };
      };
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
#pragma unroll
        for (int j = 0; j < CPW_U; ++j) {
          Uacc[i][j] *= G2;
          if constexpr (!OUT) Cacc[i][j] *= Gam;
        }
        uacc[i] *= G2;
        if constexpr (!OUT) macc[i] *= Gam;
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        frag af[RPW], aq[OUT ? 1 : RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int rb = srow(i);
          af[i] = ld_rows(KZ, LDZ, 16 * rb, kc * KR, lane);
          if (dec) af[i] = scale_frag(af[i], g, wz(kc * KR));
          if constexpr (!OUT) {
            aq[i] = ld_cols(Qs, LDK, kc * KR, 16 * rb, lane);
            if (dec) aq[i] = scale_frag(aq[i], g, wq(kc * KR));
          }
        }
#pragma unroll
        for (int j = 0; j < CPW_U; ++j) {
          const int cb = scol(j);
          if (cb < CBU) {
            frag b = ld_cols(Vs, LDV, kc * KR, 16 * cb, lane);
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              Uacc[i][j] = mma(af[i], b, Uacc[i][j]);
              if constexpr (!OUT) Cacc[i][j] = mma(aq[i], b, Cacc[i][j]);
            }
          }
        }
        if (need_den && ones_owner) {
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            uacc[i] = mma(af[i], ones, uacc[i]);
            if constexpr (!OUT) macc[i] = mma(aq[i], ones, macc[i]);
          }
        }
      }
    }
    __syncthreads();  // every read of Z, V, S0, U0 and u0 is done
    write_state();
    if (c + 1 < nch) {
      store_lds();
      if constexpr (OUT) {
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) qf[kd] = qn[kd];
      }
    }
    __syncthreads();
  }

  if constexpr (!OUT) {
    // segment summary: S | C | U | m | u
    float *sb = a.sums + ((long)bh * walk_nsum(a) + seg) * sum_block_floats(DK, DV);
    float *sS = sb, *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rb = srow(i);
#pragma unroll
      for (int j = 0; j < CPW_S; ++j) {
        const int cb = scol(j);
        if (cb < CBS) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sS[(16 * rb + 4 * g + r) * DK + 16 * cb + nl] = Sacc[i][j][r];
        }
      }
#pragma unroll
      for (int j = 0; j < CPW_U; ++j) {
        const int cb = scol(j);
        if (cb < CBU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sC[(16 * rb + 4 * g + r) * DV + 16 * cb + nl] = Cacc[i][j][r];
            sU[(16 * rb + 4 * g + r) * DV + 16 * cb + nl] = Uacc[i][j][r];
          }
        }
      }
      if (ones_owner && nl == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm[16 * rb + 4 * g + r] = need_den ? macc[i][r] : 0.f;
          su[16 * rb + 4 * g + r] = need_den ? uacc[i][r] : 0.f;
        }
      }
    }
  }
}

// Instantiate and launch one (T, DK, DV, CP) pair of walker kernels.
template <typename T, int DK, int DV, int CP>
hipError_t launch_walk_t(bool output_mode, dim3 grid, const WalkArgs &a, hipStream_t s) {
  if (output_mode)
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, CP, true>), grid, dim3(WalkCfg<T, DK, DV, CP, true>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, CP, false>), grid, dim3(WalkCfg<T, DK, DV, CP, false>::NT), 0, s,
                       a);
  return hipGetLastError();
}

}  // namespace hla2
