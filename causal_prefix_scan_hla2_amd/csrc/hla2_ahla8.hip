// hla2_ahla8.hip -- the bf16 AHLA walker with eight waves and the state in registers, for
// d <= 64 and 64 < dv <= 128 without the ratio (den neither divided by nor returned).
//
// Method (technical summary of arXiv 2510.27258 on gist.science, §2): per chunk of 64 tokens
// (local index tau) entering with the state (P0, E0), with Ad = L o D o (Q K^T) (Ad[tau][i] =
// [i <= tau] g^{tau-i} q_tau . k_i):
//   Y = diag(g^{tau+1}) Q P0 + Ad V,        O = diag(g^{tau+1}) Q E0 + Ad Y,
//   P <- g^64 P0 + K^T diag(g^{63-i}) V,   E <- g^64 E0 + K^T diag(g^{63-j}) Y,
// and in segment-summary mode also M <- M + K^T Q (no decay).
//
// Work split.  Wave w owns value column tile w (16 columns): its P and E columns (d x 16, fp32
// accumulators), and its columns of Y and of the output for all 64 tokens.  Y never leaves the
// wave's registers: the same fragments serve as the B operand of the E update (K^T Y) and as the
// A operand of the transposed output O^T = E0^T Q^T + Y^T Ad^T, so the only chunk-local product
// shared between waves is Ad, two 16 x 16 tiles per wave (token block w % 4, key blocks
// 2 (w / 4) and 2 (w / 4) + 1), which pass through LDS as rows.  The token weights of the two
// state updates are carried by a second copy of K, K~ = diag(g^{63-t}) K, formed as the rows go
// into LDS, so that neither V nor Y is weighted per wave.  Q, K, K~ and V are double-buffered in
// LDS, so the next chunk's rows go in while this chunk's are still read; the outputs are staged
// as rows (two buffers) and stored as contiguous 16-byte pieces during the next chunk.
//
// Per chunk there are two workgroup barriers:
//   [Ad -> LDS; operand fragments of V, P0, E0]
//   B1
//   [Y, outputs -> LDS (the previous chunk's stored meanwhile); P and E updates;
//    next chunk's Q, K, K~, V -> LDS]
//   B2
// As in the second-order walker, buffer loads past the end of the sequence return zero, so a
// ragged last chunk needs no special path, and no MFMA sits under a runtime branch.
#include "hla2_walk8.h"

namespace hla2 {

template <int DK, int DV, bool OUT>
struct A8Cfg {
  static constexpr int CP = 64;        // tokens per chunk
  static constexpr int NB = CP / 16;   // token blocks
  static constexpr int NW = 8;         // waves
  static constexpr int NT = 64 * NW;
  static constexpr int RT = DK / 16;   // 16-row tiles over d
  static constexpr int KD = DK / 32;   // k-steps over d
  static constexpr int KC = CP / 32;   // k-steps over chunk tokens
  static_assert(DV / 16 == NW, "one value column tile per wave");
  static_assert(RT == 4 && KD == 2, "d = 64: two key blocks of Ad per wave, two M tiles per wave");
  // Row pitches (elements), as in the second-order walker: 16-byte row reads and transpose reads
  // at 160 bytes, 8-byte row reads at 144 (Q in output mode), staged output rows at DV + 8.
  static constexpr int LDQ = OUT ? DK + 8 : DK + 16;  // Q: row reads (summary mode: also transpose reads)
  static constexpr int LDK = DK + 16;                 // K: row (and transpose) reads; K~: transpose reads
  static constexpr int LDV = DV + 16;                 // V: transpose reads
  static constexpr int LDA = CP + 16;                 // Ad rows (permuted columns, swizzled)
  static constexpr int LDO = DV + 8;                  // staged output rows
  static constexpr int NVK = CP * DK / 8 / NT;        // 16-byte vectors per thread, Q and K
  static constexpr int NVV = CP * DV / 8 / NT;        // 16-byte vectors per thread, V
  static constexpr int NPO = CP * DV / 8 / NT;        // 16-byte output pieces per thread
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + 2 * CP * LDQ;
  static constexpr int KT_OFF = K_OFF + 2 * CP * LDK;
  static constexpr int V_OFF = KT_OFF + 2 * CP * LDK;
  static constexpr int AD_OFF = V_OFF + 2 * CP * LDV;
  static constexpr int O_OFF = AD_OFF + CP * LDA;
  static constexpr int ELEMS = O_OFF + (OUT ? 2 * CP * LDO : 0);
  static constexpr int PW_OFF = ELEMS * 2;                 // bytes: decay^x, x = 0 .. 2 CP
  static constexpr int BYTES = PW_OFF + (2 * CP + 4) * 4;
  static_assert(NVK * NT * 8 == CP * DK && NVV * NT * 8 == CP * DV && NPO * NT * 8 == CP * DV, "staging split");
  static_assert(PW_OFF % 16 == 0 && BYTES <= 160 * 1024, "one workgroup's LDS");
};

// One workgroup's walk of segment `seg` of head `bh`.  Output mode starts from the segment's
// prefix (P0 | E0); with LEAD (segment 0 of a lead plan) the state after the segment is written
// as the prefix of segment 1.  Summary mode starts from zero and writes P | E | M.
template <int DK, int DV, bool OUT, bool LEAD>
__device__ __forceinline__ void ahla8_body(const AhlaArgs &a, const int bh, const int seg, unsigned char *lds) {
  using Cfg = A8Cfg<DK, DV, OUT>;
  constexpr int CP = Cfg::CP, NB = Cfg::NB, NT = Cfg::NT, RT = Cfg::RT, KD = Cfg::KD, KC = Cfg::KC;
  constexpr int LDQ = Cfg::LDQ, LDK = Cfg::LDK, LDV = Cfg::LDV, LDA = Cfg::LDA, LDO = Cfg::LDO;
  constexpr int NVK = Cfg::NVK, NVV = Cfg::NVV, NPO = Cfg::NPO;
  constexpr long PB = 2L * DK * DV, SB = 2L * DK * DV + (long)DK * DK;  // prefix and summary blocks

  bf16 *const smem = (bf16 *)lds;
  float *const pw = (float *)(lds + Cfg::PW_OFF);
  bf16 *const Qs = smem + Cfg::Q_OFF;
  bf16 *const Ks = smem + Cfg::K_OFF;
  bf16 *const Kts = smem + Cfg::KT_OFF;
  bf16 *const Vs = smem + Cfg::V_OFF;
  bf16 *const Ads = smem + Cfg::AD_OFF;
  bf16 *const Os = smem + Cfg::O_OFF;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // key-block pair and token block of the wave's Ad tiles: the second wave of SIMD w % 4 takes block
  // 3 - (w % 4), so that the tiles the causal mask zeroes whole (skipped under a wave-uniform branch)
  // are spread over the SIMDs
  const int hh = w >> 2, tb = hh ? 3 - (w & 3) : (w & 3);
  const int vc0 = 16 * w;             // first value column of the wave

  const int d = a.d, dv = a.dv;
  const int tok0 = ahla_seg_chunk0(a, seg) * CP;
  const int tokE = min(a.n, tok0 + ahla_seg_chunks(a, seg) * CP);
  const int nch = (tokE - tok0 + CP - 1) / CP;

  const long hq = (long)bh * a.n * d, hv = (long)bh * a.n * dv;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc((const bf16 *)a.q + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc((const bf16 *)a.k + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc((const bf16 *)a.v + hv, a.n * dv * 2);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc((bf16 *)a.out + hv, OUT ? a.n * dv * 2 : 0);

  for (int x = tid; x <= 2 * CP; x += NT) pw[x] = exp2f((float)x * a.log2g);

  // ---------------- staging of one chunk: global -> registers -> LDS ----------------
  u32x4 rgq[NVK], rgk[NVK], rgv[NVV];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int t0 = tok0 + c * CP;
    // padded columns read at an offset past the buffer, which returns zero
#pragma unroll
    for (int i = 0; i < NVK; ++i) {
      const int vi = tid + i * NT, t = vi / (DK / 8), e0 = 8 * (vi % (DK / 8));
      const int off = e0 < d ? ((t0 + t) * d + e0) * 2 : OOB_OFFSET;
      rgq[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      rgk[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int vi = tid + i * NT, t = vi / (DV / 8), e0 = 8 * (vi % (DV / 8));
      const int off = e0 < dv ? ((t0 + t) * dv + e0) * 2 : OOB_OFFSET;
      rgv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  };
  // the token weight g^{63-t} of each K row a thread stages (set once the decay table is in LDS)
  float ktw[NVK];
  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
    bf16 *const Qd = Qs + buf * CP * LDQ, *const Kd = Ks + buf * CP * LDK, *const Ktd = Kts + buf * CP * LDK;
    bf16 *const Vd = Vs + buf * CP * LDV;
#pragma unroll
    for (int i = 0; i < NVK; ++i) {
      const int vi = tid + i * NT, t = vi / (DK / 8), e0 = 8 * (vi % (DK / 8));
      *(u32x4 *)(Qd + t * LDQ + e0) = rgq[i];
      *(u32x4 *)(Kd + t * LDK + e0) = rgk[i];
      const bf16x8 kr = __builtin_bit_cast(bf16x8, rgk[i]);
      bf16x8 kt;
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[e] = (bf16)((float)kr[e] * ktw[i]);
      *(bf16x8 *)(Ktd + t * LDK + e0) = kt;
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int vi = tid + i * NT, t = vi / (DV / 8), e0 = 8 * (vi % (DV / 8));
      *(u32x4 *)(Vd + t * LDV + e0) = rgv[i];
    }
  };

  // ---------------- state: P, E (rows d, the wave's value columns), M (summary mode) ----------------
  // accumulator element r of tile ti holds row 16 ti + 4 g + r, column vc0 + n
  f32x4 P[RT], E[RT], M[OUT ? 1 : 2];
#pragma unroll
  for (int i = 0; i < RT; ++i) P[i] = E[i] = zero4();
  M[0] = zero4();
  if constexpr (!OUT) M[1] = zero4();
  // with a prologue fold (below) segment 2 starts from segment 1's prefix
  const bool pfold = OUT && !LEAD && a.pfold && seg == 2;
  if (OUT && seg > 0) {
    const float *pref = a.prefix + ((long)bh * a.nseg + (pfold ? 1 : seg)) * PB;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        P[i][r] = pref[(16 * i + 4 * g + r) * DV + vc0 + n];
        E[i][r] = pref[DK * DV + (16 * i + 4 * g + r) * DV + vc0 + n];
      }
  }

  load_chunk(0);

  // Prologue fold (a three-segment lead plan has no scan launch): segment 2 folds segment 1's
  // summary (P_1, E_1, M_1) onto segment 1's prefix with the scan's combine,
  //   E <- G E + E_1 + G M_1 P,   P <- G P + P_1   (G = decay^(tokens per segment)),
  // M_1 P on bf16 MFMA with M_1's rows read straight from the summary and P from registers,
  // while the first chunk's rows are in flight.
  if constexpr (OUT && !LEAD) {
    if (pfold) {
      const float G = a.gseg;
      const float *sb = a.sums + ((long)bh * (a.nseg - 1) + 1) * SB, *M1 = sb + 2 * DK * DV;
      bf16x8 pb[KD];
#pragma unroll
      for (int s = 0; s < KD; ++s) pb[s] = frag_from_acc(P[2 * s], P[2 * s + 1]);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        f32x4 x = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) {
          // M_1 rows 16 i + n, columns of the accumulator k-order of lane group g
          const float *mr = M1 + (16 * i + n) * DK + 32 * s + 4 * g;
          const f32x4 lo = *(const f32x4 *)mr, hi = *(const f32x4 *)(mr + 16);
          x = mma(frag_from_acc(lo, hi), pb[s], x);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
          E[i][r] = G * E[i][r] + sb[DK * DV + o] + G * x[r];
          P[i][r] = G * P[i][r] + sb[o];
        }
      }
    }
  }

  // ---------------- loop-invariant factors ----------------
  __syncthreads();  // pw
  const int tau_w = 16 * tb + n;  // this lane's row of the wave's Ad tiles
  // Ad^T tile 2 hh + jj of block tb: element r is (i = 16 (2 hh + jj) + 4 g + r, tau = tau_w),
  // weight [i <= tau] g^{tau - i}
  float fa[2][4];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * (tb - 2 * hh - jj) + n - 4 * g - r;
      fa[jj][r] = e >= 0 ? pw[e] : 0.f;
    }
#pragma unroll
  for (int i = 0; i < NVK; ++i) ktw[i] = pw[CP - 1 - (tid + i * NT) / (DK / 8)];
  const float gC = pw[CP];
  // g^{tau+1} of the Y tile rows (tau = 16 r + 4 g + q) and of the transposed output columns
  // (tau = 16 r + n)
  float yf[NB][4], of[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    of[r] = pw[16 * r + n + 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) yf[r][q] = pw[16 * r + 4 * g + q + 1];
  }

  // Staged outputs: the rows a chunk left in its output buffer, from token trow on, as contiguous
  // 16-byte pieces (lanes 0-7 and 16-23 take one whole row, so that a read covers the 64 banks
  // once).  A row base of n drops every store.
  auto flush_out = [&](int trow, int obuf) __attribute__((always_inline)) {
    if constexpr (OUT) {
      const bf16 *const Ob = Os + obuf * CP * LDO;
#pragma unroll
      for (int i = 0; i < NPO; ++i) {
        const int id = tid + i * NT, l = id & 31;
        const int row = 2 * (id >> 5) + ((l >> 3) & 1);
        const int cg = 8 * ((l & 7) | ((l >> 4) << 3));
        const u32x4 x = *(const u32x4 *)(Ob + row * LDO + cg);
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, cg < dv ? ((trow + row) * dv + cg) * 2 : 0x7fffffff, 0, 0);
      }
    }
  };

  store_chunk(0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bf16 *const Qc = Qs + buf * CP * LDQ, *const Kc = Ks + buf * CP * LDK, *const Vc = Vs + buf * CP * LDV;
    const bf16 *const Ktc = Kts + buf * CP * LDK;
    bf16 *const Oc = Os + buf * CP * LDO;
    // the next chunk's loads fly during phase 1 (a repeat of the last chunk at the end; it is
    // never read)
    load_chunk(min(c + 1, nch - 1));
    __builtin_amdgcn_sched_barrier(0);

    // ======== phase 1 ========
    // Ad^T tiles of the wave (rows i, column tau) -> masked, decayed -> one 16-byte piece of
    // Ad row tau_w: tiles 2 hh and 2 hh + 1 side by side in the accumulator k-order (w8_wpos)
    {
      bf16x8 qw[KD];
#pragma unroll
      for (int s = 0; s < KD; ++s) qw[s] = w8_rows(Qc, LDQ, 16 * tb, 32 * s, lane);
      f32x4 at[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        at[jj] = zero4();
        if (2 * hh + jj <= tb) {
#pragma unroll
          for (int s = 0; s < KD; ++s) at[jj] = mma(w8_rows(Kc, LDK, 16 * (2 * hh + jj), 32 * s, lane), qw[s], at[jj]);
#pragma unroll
          for (int r = 0; r < 4; ++r) at[jj][r] *= fa[jj][r];
        }
      }
      *(bf16x8 *)(Ads + tau_w * LDA + ((32 * hh + 8 * g) ^ w8_swl(lane))) =
          bf16x8{(bf16)at[0][0], (bf16)at[0][1], (bf16)at[0][2], (bf16)at[0][3],
                 (bf16)at[1][0], (bf16)at[1][1], (bf16)at[1][2], (bf16)at[1][3]};
    }

    // V columns of the wave (B operand of Y = Ad V and of the P update)
    bf16x8 vf[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) vf[s] = ld_cols(Vc, LDV, 32 * s, vc0, lane);
    // P0 and E0 fragments (B operands of Q P0 and, transposed, of E0^T Q^T), taken before the updates
    bf16x8 p0b[KD], e0b[OUT ? KD : 1];
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      p0b[s] = frag_from_acc(P[2 * s], P[2 * s + 1]);
      if constexpr (OUT) e0b[s] = frag_from_acc(E[2 * s], E[2 * s + 1]);
    }
    if constexpr (!OUT) {
      // M <- M + K^T Q: tiles (row tile w / 2, column tiles 2 (w % 2) + jj)
      bf16x8 mk[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) mk[s] = ld_cols(Kc, LDK, 32 * s, 16 * (w >> 1), lane);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int s = 0; s < KC; ++s) M[jj] = mma(mk[s], ld_cols(Qc, LDQ, 32 * s, 16 * (2 * (w & 1) + jj), lane), M[jj]);
    }

    __syncthreads();  // B1: Ad visible

    // ======== phase 2 ========
    // Ordered for independent MFMA chains: the carried-state products of all four token blocks
    // (Q P0 and E0^T Q^T) and the P update (neither waits for Y), then the chunk-local terms.
    // Ad row fragments (accumulator k-order) of the needed k-steps (block r reads keys below
    // 16 r + 16: k-step s when 32 s <= 16 r + 15), and Q row fragments in the accumulator
    // k-order (A operand of Q P0, B operand of E0^T Q^T)
    bf16x8 ad[NB][KC], qa[NB][KD];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
#pragma unroll
      for (int s = 0; s < KD; ++s) qa[r][s] = w8_rows_acc(Qc, LDQ, 16 * r, 32 * s, lane);
#pragma unroll
      for (int s = 0; s < KC; ++s)
        if (32 * s <= 16 * r + 15) ad[r][s] = w8_rows_sw(Ads, LDA, 16 * r, 32 * s, lane);
    }
    // Y tiles (rows tau, the wave's columns) = diag(g^{tau+1}) Q P0 + Ad V, and the transposed
    // outputs (rows = the wave's value columns, columns = tau) O^T = diag(g^{tau+1}) E0^T Q^T +
    // Y^T Ad^T: first the carried-state terms
    f32x4 Y[NB], O[OUT ? NB : 1];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      Y[r] = zero4();
#pragma unroll
      for (int s = 0; s < KD; ++s) Y[r] = mma(qa[r][s], p0b[s], Y[r]);
    }
    if constexpr (OUT) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        O[r] = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) O[r] = mma(e0b[s], qa[r][s], O[r]);
      }
    }
    // P <- g^64 P + K~^T V  (K~ = diag(g^{63-t}) K); the K~ fragments stay for the E update
    bf16x8 kt[RT][KC];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
      for (int s = 0; s < KC; ++s) kt[i][s] = ld_cols(Ktc, LDK, 32 * s, 16 * i, lane);
      f32x4 pa = gC * P[i];
#pragma unroll
      for (int s = 0; s < KC; ++s) pa = mma(kt[i][s], vf[s], pa);
      P[i] = pa;
    }
    // the chunk-local term of Y
#pragma unroll
    for (int r = 0; r < NB; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q) Y[r][q] *= yf[r][q];
#pragma unroll
      for (int s = 0; s < KC; ++s)
        if (32 * s <= 16 * r + 15) Y[r] = mma(ad[r][s], vf[s], Y[r]);
    }
    // Y fragments over tokens (accumulator k-order): A operand of Y^T Ad^T, B operand of the E
    // update
    bf16x8 yb[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) yb[s] = frag_from_acc(Y[2 * s], Y[2 * s + 1]);
    // the chunk-local term of the outputs, staged as rows
    if constexpr (OUT) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        f32x4 o = O[r] * of[r];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          if (32 * s <= 16 * r + 15) o = mma(yb[s], ad[r][s], o);
        *(bf16x4 *)(Oc + (16 * r + n) * LDO + vc0 + 4 * g) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
      }
    }
    // E <- g^64 E + K~^T Y
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      f32x4 ea = gC * E[i];
#pragma unroll
      for (int s = 0; s < KC; ++s) ea = mma(kt[i][s], yb[s], ea);
      E[i] = ea;
    }
    // the previous chunk's staged outputs (none before the first chunk: row base n), issued
    // after the next chunk's loads
    flush_out(__builtin_amdgcn_readfirstlane(c > 0 ? tok0 + (c - 1) * CP : a.n), buf ^ 1);
    // the next chunk's rows into the other buffer (read last in the previous chunk, which every
    // wave finished before B1)
    store_chunk(buf ^ 1);

    __syncthreads();  // B2: the outputs and the next chunk's rows visible; every read of Ad done
  }
  // the last chunk's outputs (visible after B2)
  if constexpr (OUT) {
    if (nch > 0) flush_out(tok0 + (nch - 1) * CP, (nch - 1) & 1);
  }

  // ---------------- segment summary: P | E | M ----------------
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * (a.nseg - 1) + seg) * SB;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
        sb[o] = P[i][r];
        sb[DK * DV + o] = E[i][r];
      }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sb[2 * DK * DV + (16 * (w >> 1) + 4 * g + r) * DK + 16 * (2 * (w & 1) + jj) + n] = M[jj][r];
  }
  // ---------------- lead segment: its final state is the prefix of segment 1 ----------------
  if constexpr (OUT && LEAD) {
    float *pb = a.prefix + ((long)bh * a.nseg + seg + 1) * PB;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
        pb[o] = P[i][r];
        pb[DK * DV + o] = E[i][r];
      }
  }
}

// Walks segments (OUT ? seg_lo .. nseg-1 : 0 .. nseg-2) of every head, one workgroup each; one
// workgroup of eight waves per CU.
template <int DK, int DV, bool OUT>
__global__ void __launch_bounds__(512, 2) ahla8_walk_kernel(AhlaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[A8Cfg<DK, DV, OUT>::BYTES];
  const int lo = OUT ? a.seg_lo : 0, nr = (OUT ? a.nseg : a.nseg - 1) - lo;
  ahla8_body<DK, DV, OUT, false>(a, blockIdx.x / nr, lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head for its outputs and leave
// the prefix of segment 1; the rest summarise segments 1 .. nseg-2 of every head.  Both roles
// share one LDS allocation (the larger, output mode's).
template <int DK, int DV>
__global__ void __launch_bounds__(512, 2) ahla8_lead_kernel(AhlaArgs a) {
  constexpr int BO = A8Cfg<DK, DV, true>::BYTES, BS = A8Cfg<DK, DV, false>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[BO > BS ? BO : BS];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    ahla8_body<DK, DV, true, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = a.nseg - 2;
    ahla8_body<DK, DV, false, false>(a, i / nr, 1 + i % nr, lds);
  }
}

hipError_t launch_ahla8(int phase, int BH, const AhlaArgs &a, hipStream_t s) {
  if (a.kc != 64) return hipErrorInvalidValue;
  switch (phase) {
    case AHLA_SUMMARY:
      hipLaunchKernelGGL((ahla8_walk_kernel<64, 128, false>), dim3(BH * (a.nseg - 1)), dim3(512), 0, s, a);
      return hipGetLastError();
    case AHLA_OUTPUT:
      hipLaunchKernelGGL((ahla8_walk_kernel<64, 128, true>), dim3(BH * (a.nseg - a.seg_lo)), dim3(512), 0, s, a);
      return hipGetLastError();
    case AHLA_LEAD:
      if (a.nseg < 2 || a.nbh != BH) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ahla8_lead_kernel<64, 128>), dim3(BH * (a.nseg - 1)), dim3(512), 0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace hla2
