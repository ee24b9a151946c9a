// hla2_ho38.hip -- the bf16 third-order walker with eight waves and the state in registers, for
// d <= 64 and 64 < dv <= 128 without the ratio (den neither divided by nor returned).
//
// Method (technical summary of arXiv 2510.27258 on gist.science, §3, in the masked reading of the
// tile walker in hla2_ho3.hip): per chunk of 64 tokens (local index tau) entering with the state
// (S0, P0, W0), with Ad = L o D o (Q K^T) (Ad[tau][i] = [i <= tau] g^{tau-i} q_tau . k_i) and
// Wm = L o D3 o (Q Z^T) (Wm[tau][l] = [l <= tau] g^{3(tau-l)} q_tau . z_l):
//   Z = diag(g^{tau+1}) Q S0 + Ad K,       Y = diag(g^{tau+1}) Q P0 + Ad V,
//   O = diag(g^{3(tau+1)}) Q W0 + Wm Y,
//   S <- g^64 S0 + K^T diag(g^{63-i}) K,   P <- g^64 P0 + K^T diag(g^{63-i}) V,
//   W <- g^192 W0 + Z^T diag(g^{3(63-l)}) Y,
// and in segment-summary mode the segment maps (u = the token's index in its segment of L tokens)
//   Q2 += sum_u g^{3L-1-u} q_u q_u^T,  X1 += sum_u g^{3L-2-2u} q_u y_u^T,  X2 += sum_u g^{3L-2-2u} z_u q_u^T.
//
// Work split.  The d-space part is the second-order walker's (hla2_walk8.h): wave w = 4 h + b forms
// the four Ad^T tiles of token block b, the Z^T tiles of d-row tiles 2h, 2h+1 of that block, its S
// tiles, and the Wm^T tiles of key blocks 2h, 2h+1; Z, its decayed copy Z~ and Wm pass through LDS as
// rows.  The value part is the AHLA walker's (hla2_ahla8.hip): wave w owns value column tile w, with
// its columns of P and W in fp32 accumulators and its columns of Y for all 64 tokens in registers;
// Y is formed untransposed, so that a pair of its accumulator tiles is the token-ordered fragment
// that the W update, the output O^T = W0^T Q^T + Y^T Wm^T and the map X1 all take.  Each wave also
// writes two of its Ad^T tiles as Ad rows, which every wave reads for Y.  The token weights of the S
// and P updates ride on a second copy of K, K~ = diag(g^{63-t}) K, formed as the rows go into LDS.
//
// Per chunk there are two workgroup barriers, as in the second-order walker:
//   [Ad, Z, Z~ -> LDS; S and P updates; operand fragments]
//   B1
//   [S0, next chunk's rows -> LDS; Wm -> LDS; Y; W update; maps (summary mode)]
//   B2
//   [outputs]
// Buffer loads past the end of the sequence return zero, so a ragged last chunk needs no special
// path, and no MFMA sits under a runtime branch.
#include "hla2_walk8.h"

namespace hla2 {

template <int DK, int DV, bool OUT>
struct H8Cfg {
  static constexpr int CP = 64;        // tokens per chunk
  static constexpr int NB = CP / 16;   // token blocks
  static constexpr int NW = 8;         // waves
  static constexpr int NT = 64 * NW;
  static constexpr int RT = DK / 16;   // 16-row tiles over d
  static constexpr int KD = DK / 32;   // k-steps over d
  static constexpr int KC = CP / 32;   // k-steps over chunk tokens
  static constexpr int SRT = RT / 2;   // S (and Z^T) d-row tiles per wave
  static constexpr int SCT = RT / 4;   // S column tiles per wave
  static_assert(DV / 16 == NW, "one value column tile per wave");
  static_assert(RT == 4 && KD == 2 && SCT == 1, "d = 64");
  // Row pitches (elements), as in the second-order walker: 16-byte row reads and transpose reads at
  // 160 bytes, 8-byte row reads at 144 (Q in output mode), staged output rows at DV + 8.  Z~, S0, Z,
  // Ad and Wm take 8- or 16-byte row writes from accumulator tiles and are swizzled (w8_swl).
  static constexpr int LDQ = OUT ? DK + 8 : DK + 16;  // Q: row reads (summary mode: also transpose reads)
  static constexpr int LDK = DK + 16;                 // K, K~: row and transpose reads
  static constexpr int LDV = DV + 16;                 // V: transpose reads
  static constexpr int LDT = DK + 16;                 // Z~: transpose reads
  static constexpr int LDS0 = DK + 16;                // S0: row reads
  static constexpr int LDZ = DK + 16;                 // Z: row reads (summary mode: also transpose reads)
  static constexpr int LDA = CP + 16;                 // Ad rows (permuted columns)
  static constexpr int LDW = CP + 16;                 // Wm rows (permuted columns)
  static constexpr int LDO = DV + 8;                  // staged output rows
  static constexpr int NVK = CP * DK / 8 / NT;        // 16-byte vectors per thread, Q and K
  static constexpr int NVV = CP * DV / 8 / NT;        // 16-byte vectors per thread, V
  static constexpr int NPO = CP * DV / 8 / NT;        // 16-byte output pieces per thread
  static constexpr int Q_OFF = 0;                     // two buffers: Q is read until the chunk's end
  static constexpr int K_OFF = Q_OFF + 2 * CP * LDQ;
  static constexpr int KT_OFF = K_OFF + CP * LDK;
  static constexpr int V_OFF = KT_OFF + CP * LDK;
  static constexpr int ZT_OFF = V_OFF + CP * LDV;
  static constexpr int SB_OFF = ZT_OFF + CP * LDT;
  static constexpr int Z_OFF = SB_OFF + DK * LDS0;
  static constexpr int AD_OFF = Z_OFF + CP * LDZ;
  static constexpr int W_OFF = AD_OFF + CP * LDA;
  static constexpr int O_OFF = W_OFF + (OUT ? CP * LDW : 0);
  static constexpr int ELEMS = O_OFF + (OUT ? CP * LDO : 0);
  static constexpr int PW_OFF = ELEMS * 2;            // bytes: decay^x, x = 0 .. 3 CP
  static constexpr int BYTES = PW_OFF + (3 * CP + 4) * 4;
  static_assert(NVK * NT * 8 == CP * DK && NVV * NT * 8 == CP * DV && NPO * NT * 8 == CP * DV, "staging split");
  static_assert(PW_OFF % 16 == 0 && BYTES <= 160 * 1024, "one workgroup's LDS");
};

// One workgroup's walk of segment `seg` of head `bh`.  Output mode starts from the segment's prefix
// S0 | P0 | W0; with LEAD (segment 0 of a lead plan) the state after the segment is written as the
// prefix of segment 1.  Summary mode starts from zero and writes S | P | W | Q2 | X1 | X2.
template <int DK, int DV, bool OUT, bool LEAD>
__device__ __forceinline__ void ho38_body(const Ho3Args &a, const int bh, const int seg, unsigned char *lds) {
  using Cfg = H8Cfg<DK, DV, OUT>;
  constexpr int CP = Cfg::CP, NB = Cfg::NB, NT = Cfg::NT, RT = Cfg::RT, KD = Cfg::KD, KC = Cfg::KC;
  constexpr int SRT = Cfg::SRT, SCT = Cfg::SCT;
  constexpr int LDQ = Cfg::LDQ, LDK = Cfg::LDK, LDV = Cfg::LDV, LDT = Cfg::LDT, LDS0 = Cfg::LDS0;
  constexpr int LDZ = Cfg::LDZ, LDA = Cfg::LDA, LDW = Cfg::LDW, LDO = Cfg::LDO;
  constexpr int NVK = Cfg::NVK, NVV = Cfg::NVV, NPO = Cfg::NPO;
  constexpr long PB = (long)DK * DK + 2L * DK * DV;       // prefix block S | P | W
  constexpr long SB = PB + 2L * DK * DK + (long)DK * DV;  // summary block: ... | Q2 | X1 | X2

  bf16 *const smem = (bf16 *)lds;
  float *const pw = (float *)(lds + Cfg::PW_OFF);
  bf16 *const Qs = smem + Cfg::Q_OFF;
  bf16 *const Ks = smem + Cfg::K_OFF;
  bf16 *const Kts = smem + Cfg::KT_OFF;
  bf16 *const Vs = smem + Cfg::V_OFF;
  bf16 *const Zts = smem + Cfg::ZT_OFF;
  bf16 *const Sb = smem + Cfg::SB_OFF;
  bf16 *const Zs = smem + Cfg::Z_OFF;
  bf16 *const Ads = smem + Cfg::AD_OFF;
  bf16 *const Wms = smem + Cfg::W_OFF;
  bf16 *const Os = smem + Cfg::O_OFF;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // half and token block.  In output mode the second wave of SIMD w % 4 takes block 3 - (w % 4), so
  // every SIMD holds one block near the chunk's start and one near its end, and the products over key
  // blocks that the causal mask zeroes whole (A, Z, Wm) are skipped under wave-uniform branches.  The
  // summary walk keeps block w % 4 and computes them (the skip measured slower there).
  constexpr bool CS = OUT;
  const int hh = w >> 2, tb = (CS && hh) ? 3 - (w & 3) : (w & 3);
  const int srow0 = hh * SRT;         // first d-row tile of the wave's S and Z^T tiles
  const int scol0 = tb * SCT;         // column tile of the wave's S tile
  const int vc0 = 16 * w;             // first value column of the wave
  const int mti = w >> 1;             // summary maps Q2, X2: row tile, column tiles 2 (w % 2) + jj
  const int mtj0 = 2 * (w & 1);

  const int d = a.d, dv = a.dv;
  const int tok0 = ahla_seg_chunk0(a, seg) * CP;
  const int tokE = min(a.n, tok0 + ahla_seg_chunks(a, seg) * CP);
  const int nch = (tokE - tok0 + CP - 1) / CP;
  const int seglen = a.cps * CP;  // summarised segments are full (segment 0 of a lead plan is never summarised)

  const long hq = (long)bh * a.n * d, hv = (long)bh * a.n * dv;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc((const bf16 *)a.q + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc((const bf16 *)a.k + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc((const bf16 *)a.v + hv, a.n * dv * 2);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc((bf16 *)a.out + hv, OUT ? a.n * dv * 2 : 0);

  for (int x = tid; x <= 3 * CP; x += NT) pw[x] = exp2f((float)x * a.log2g);

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
  auto store_chunk = [&](int qbuf) __attribute__((always_inline)) {
    bf16 *const Qd = Qs + qbuf * CP * LDQ;
#pragma unroll
    for (int i = 0; i < NVK; ++i) {
      const int vi = tid + i * NT, t = vi / (DK / 8), e0 = 8 * (vi % (DK / 8));
      *(u32x4 *)(Qd + t * LDQ + e0) = rgq[i];
      *(u32x4 *)(Ks + t * LDK + e0) = rgk[i];
      const bf16x8 kr = __builtin_bit_cast(bf16x8, rgk[i]);
      bf16x8 kt;
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[e] = (bf16)((float)kr[e] * ktw[i]);
      *(bf16x8 *)(Kts + t * LDK + e0) = kt;
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int vi = tid + i * NT, t = vi / (DV / 8), e0 = 8 * (vi % (DV / 8));
      *(u32x4 *)(Vs + t * LDV + e0) = rgv[i];
    }
  };

  // ---------------- state ----------------
  // S tile (i, j): rows 16 (srow0 + i) + 4 g + r, column 16 (scol0 + j) + n; P and W tile ti: rows
  // 16 ti + 4 g + r, column vc0 + n
  f32x4 Sacc[SRT][SCT], P[RT], W[RT];
  f32x4 Q2m[OUT ? 1 : 2], X2m[OUT ? 1 : 2], X1m[OUT ? 1 : RT];
#pragma unroll
  for (int i = 0; i < SRT; ++i)
#pragma unroll
    for (int j = 0; j < SCT; ++j) Sacc[i][j] = zero4();
#pragma unroll
  for (int i = 0; i < RT; ++i) P[i] = W[i] = zero4();
  if constexpr (!OUT) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) Q2m[jj] = X2m[jj] = zero4();
#pragma unroll
    for (int i = 0; i < RT; ++i) X1m[i] = zero4();
  }
  // with a prologue fold (below) segment 2 starts from segment 1's prefix
  const bool pfold = OUT && !LEAD && a.pfold && seg == 2;
  const float *const pref = (OUT && seg > 0) ? a.prefix + ((long)bh * a.nseg + (pfold ? 1 : seg)) * PB : nullptr;
  if (OUT && seg > 0) {
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[i][j][r] = pref[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
        P[i][r] = pref[DK * DK + o];
        W[i][r] = pref[DK * DK + DK * DV + o];
      }
  }
  // S0 as bf16 rows (S is symmetric: each tile is written transposed, as rows of its column)
  auto write_S0 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
        st4(Sb + (16 * (scol0 + j) + n) * LDS0 + 16 * (srow0 + i) + ((4 * g) ^ w8_swl(lane)), Sacc[i][j]);
  };

  load_chunk(0);

  // Prologue fold (a three-segment lead plan has no scan launch): segment 2 folds segment 1's
  // summary (S_1, P_1, W_1, Q2, X1, X2) onto segment 1's prefix (S_A, P_A, W_A) with the segment
  // combine
  //   T = S_A Q2 + X2,   W <- G^3 W_A + W_1 + T P_A + S_A X1,   S <- G S_A + S_1,   P <- G P_A + P_1
  // (G = decay^(tokens per segment)), on bf16 MFMA with every operand read straight from global
  // memory into fragments (P_A from the accumulators), while the first chunk's rows are in flight.
  // Each wave forms all of T, as T^T tiles, whose accumulator pairs are T's row fragments.
  if constexpr (OUT && !LEAD) {
    if (pfold) {
      const float G = a.gseg, G3 = G * G * G;
      const float *sb = a.sums + ((long)bh * (a.nseg - 1) + 1) * SB;
      const float *Q2g = sb + PB, *X1g = Q2g + DK * DK, *X2g = X1g + DK * DV;
      // S_A row fragments: lane (g, n) of (I, s) holds S_A[16 I + n][32 s + 4 g + 0..3, + 16 + 0..3]
      bf16x8 sa[RT][KD];
#pragma unroll
      for (int I = 0; I < RT; ++I)
#pragma unroll
        for (int s = 0; s < KD; ++s) {
          const float *p = pref + (16 * I + n) * DK + 32 * s + 4 * g;
          sa[I][s] = frag_from_acc(*(const f32x4 *)p, *(const f32x4 *)(p + 16));
        }
      // T^T tile (J, I) = Q2^T S_A^T + X2^T: lane (g, n) element r is T[16 I + n][16 J + 4 g + r]
      bf16x8 tf[RT][KD];
#pragma unroll
      for (int I = 0; I < RT; ++I) {
        f32x4 tt[RT];
#pragma unroll
        for (int J = 0; J < RT; ++J) {
          tt[J] = *(const f32x4 *)(X2g + (16 * I + n) * DK + 16 * J + 4 * g);
#pragma unroll
          for (int s = 0; s < KD; ++s) {
            // Q2 columns 16 J + n, rows of the accumulator k-order of lane group g
            bf16x8 qc;
#pragma unroll
            for (int e = 0; e < 8; ++e) qc[e] = (bf16)Q2g[(32 * s + kidx<bf16>(g, e)) * DK + 16 * J + n];
            tt[J] = mma(qc, sa[I][s], tt[J]);
          }
        }
#pragma unroll
        for (int s = 0; s < KD; ++s) tf[I][s] = frag_from_acc(tt[2 * s], tt[2 * s + 1]);
      }
      bf16x8 pb[KD], xb[KD];
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        pb[s] = frag_from_acc(P[2 * s], P[2 * s + 1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[s][e] = (bf16)X1g[(32 * s + kidx<bf16>(g, e)) * DV + vc0 + n];
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        f32x4 x = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) {
          x = mma(tf[i][s], pb[s], x);
          x = mma(sa[i][s], xb[s], x);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
          W[i][r] = G3 * W[i][r] + sb[DK * DK + DK * DV + o] + x[r];
          P[i][r] = G * P[i][r] + sb[DK * DK + o];
        }
      }
#pragma unroll
      for (int i = 0; i < SRT; ++i)
#pragma unroll
        for (int j = 0; j < SCT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Sacc[i][j][r] = G * Sacc[i][j][r] + sb[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n];
    }
  }

  // ---------------- loop-invariant factors ----------------
  __syncthreads();  // pw
  const int tau_w = 16 * tb + n;  // this lane's column in the wave's Ad^T, Z^T and Wm^T tiles
  // Ad^T tile I of the wave's block: element r is (i = 16 I + 4 g + r, tau = tau_w), weight
  // [i <= tau] g^{tau - i}; Wm^T tiles J = 2 h + jj: [l <= tau] g^{3 (tau - l)}
  float fa[NB][4], fw[2][4];
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * (tb - I) + n - 4 * g - r;
      fa[I][r] = e >= 0 ? pw[e] : 0.f;
    }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * (tb - 2 * hh - jj) + n - 4 * g - r;
      fw[jj][r] = e >= 0 ? pw[3 * e] : 0.f;
    }
#pragma unroll
  for (int i = 0; i < NVK; ++i) ktw[i] = pw[CP - 1 - (tid + i * NT) / (DK / 8)];
  const float zf = pw[tau_w + 1];               // g^{tau+1} (Z)
  const float ztf = pw[3 * (CP - 1 - tau_w)];   // g^{3(63-tau)} (Z~)
  const float g64 = pw[CP], g192 = pw[3 * CP];
  // g^{tau+1} of the Y tile rows (tau = 16 r + 4 g + q) and g^{3(tau+1)} of the transposed output
  // columns (tau = 16 r + n)
  float yf[NB][4], of[OUT ? NB : 1];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    if constexpr (OUT) of[r] = pw[3 * (16 * r + n + 1)];
#pragma unroll
    for (int q = 0; q < 4; ++q) yf[r][q] = pw[16 * r + 4 * g + q + 1];
  }

  // Staged outputs: the rows phase 3 left in LDS, from token trow on, as contiguous 16-byte pieces
  // (lanes 0-7 and 16-23 take one whole row, so that a read covers the 64 banks once), issued after
  // the barrier that follows the next chunk's loads.  A row base of n drops every store.
  auto flush_out = [&](int trow) __attribute__((always_inline)) {
    if constexpr (OUT) {
#pragma unroll
      for (int i = 0; i < NPO; ++i) {
        const int id = tid + i * NT, l = id & 31;
        const int row = 2 * (id >> 5) + ((l >> 3) & 1);
        const int cg = 8 * ((l & 7) | ((l >> 4) << 3));
        const u32x4 x = *(const u32x4 *)(Os + row * LDO + cg);
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, cg < dv ? ((trow + row) * dv + cg) * 2 : 0x7fffffff, 0, 0);
      }
    }
  };

  write_S0();
  store_chunk(0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const bf16 *const Qc = Qs + (c & 1) * CP * LDQ;  // this chunk's Q
    // the next chunk's loads fly during phase 1 and land in LDS after B1 (a repeat of the last
    // chunk at the end; it is never read)
    load_chunk(min(c + 1, nch - 1));
    __builtin_amdgcn_sched_barrier(0);

    // ======== phase 1 ========
    bf16x8 qw[KD];
#pragma unroll
    for (int s = 0; s < KD; ++s) qw[s] = w8_rows(Qc, LDQ, 16 * tb, 32 * s, lane);
    // Ad^T tiles of the wave's block (rows i, column tau), masked and decayed: fragments for Z, and
    // the key blocks 2 h, 2 h + 1 as one 16-byte piece of Ad row tau_w (accumulator k-order, w8_wpos)
    bf16x8 adf[KC];
    {
      f32x4 at[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        at[I] = zero4();
        if (!CS || I <= tb) {  // key blocks after the wave's block are masked whole
#pragma unroll
          for (int s = 0; s < KD; ++s) at[I] = mma(w8_rows(Ks, LDK, 16 * I, 32 * s, lane), qw[s], at[I]);
#pragma unroll
          for (int r = 0; r < 4; ++r) at[I][r] *= fa[I][r];
        }
      }
#pragma unroll
      for (int s = 0; s < KC; ++s) adf[s] = frag_from_acc(at[2 * s], at[2 * s + 1]);
      *(bf16x8 *)(Ads + tau_w * LDA + ((32 * hh + 8 * g) ^ w8_swl(lane))) = hh ? adf[1] : adf[0];
    }
    // per d-row tile ti of the wave, with the K^T fragments of that tile (A operand, k = tokens):
    //   Z^T tile (rows d, column tau): S0 Q_b^T scaled by g^{tau+1}, plus K^T Ad_b^T, as Z and Z~ rows;
    //   S <- g^64 S + K^T diag(g^{63-t}) K on the wave's S tiles in that row tile (K~ columns).
#pragma unroll
    for (int i = 0; i < SRT; ++i) {
      const int ti = srow0 + i;
      bf16x8 kt[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) kt[s] = ld_cols(Ks, LDK, 32 * s, 16 * ti, lane);
      f32x4 z = zero4();
#pragma unroll
      for (int s = 0; s < KD; ++s) z = mma(w8_rows_sw(Sb, LDS0, 16 * ti, 32 * s, lane), qw[s], z);
      z *= zf;
#pragma unroll
      for (int s = 0; s < KC; ++s)
        if (!CS || 32 * s <= 16 * tb + 15) z = mma(kt[s], adf[s], z);
      st4(Zs + tau_w * LDZ + 16 * ti + ((4 * g) ^ w8_swl(lane)), z);
      st4(Zts + tau_w * LDT + 16 * ti + ((4 * g) ^ w8_swl(lane)), z * ztf);
#pragma unroll
      for (int j = 0; j < SCT; ++j) {
        f32x4 acc = Sacc[i][j] * g64;
#pragma unroll
        for (int s = 0; s < KC; ++s) acc = mma(kt[s], ld_cols(Kts, LDK, 32 * s, 16 * (scol0 + j), lane), acc);
        Sacc[i][j] = acc;
      }
    }
    // V columns of the wave (B operand of Y = Ad V and of the P update)
    bf16x8 vf[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) vf[s] = ld_cols(Vs, LDV, 32 * s, vc0, lane);
    // P0 and W0 fragments (B operand of Q P0; A operand of W0^T Q^T), taken before the updates
    bf16x8 p0b[KD], w0b[OUT ? KD : 1];
#pragma unroll
    for (int s = 0; s < KD; ++s) {
      p0b[s] = frag_from_acc(P[2 * s], P[2 * s + 1]);
      if constexpr (OUT) w0b[s] = frag_from_acc(W[2 * s], W[2 * s + 1]);
    }
    // P <- g^64 P + K~^T V
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      f32x4 acc = P[i] * g64;
#pragma unroll
      for (int s = 0; s < KC; ++s) acc = mma(ld_cols(Kts, LDK, 32 * s, 16 * i, lane), vf[s], acc);
      P[i] = acc;
    }

    __syncthreads();  // B1: Ad, Z, Z~ visible; every read of this chunk's K, K~, V and S0 is done

    // ======== phase 2 ========
    // the previous chunk's staged outputs (none before the first chunk: row base n)
    flush_out(__builtin_amdgcn_readfirstlane(c > 0 ? tok0 + (c - 1) * CP : a.n));
    write_S0();
    store_chunk((c + 1) & 1);

    if constexpr (OUT) {
      // Wm^T tiles J = 2h, 2h+1 of the block (rows l, column tau) -> masked, decayed -> Wm rows
      f32x4 wt[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = 2 * hh + jj;
        wt[jj] = zero4();
        if (!CS || J <= tb) {
#pragma unroll
          for (int s = 0; s < KD; ++s) wt[jj] = mma(w8_rows_sw(Zs, LDZ, 16 * J, 32 * s, lane), qw[s], wt[jj]);
#pragma unroll
          for (int r = 0; r < 4; ++r) wt[jj][r] *= fw[jj][r];
        }
      }
      *(bf16x8 *)(Wms + tau_w * LDW + ((32 * hh + 8 * g) ^ w8_swl(lane))) =
          bf16x8{(bf16)wt[0][0], (bf16)wt[0][1], (bf16)wt[0][2], (bf16)wt[0][3],
                 (bf16)wt[1][0], (bf16)wt[1][1], (bf16)wt[1][2], (bf16)wt[1][3]};
    }
    // Y tiles (rows tau, the wave's columns) = diag(g^{tau+1}) Q P0 + Ad V: the carried-state terms
    // of all four token blocks first (independent chains), then the chunk-local ones
    f32x4 Y[NB];
    {
      bf16x8 qa[NB][KD];
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        Y[r] = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) {
          qa[r][s] = w8_rows_acc(Qc, LDQ, 16 * r, 32 * s, lane);
          Y[r] = mma(qa[r][s], p0b[s], Y[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < NB; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) Y[r][q] *= yf[r][q];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          if (32 * s <= 16 * r + 15) Y[r] = mma(w8_rows_sw(Ads, LDA, 16 * r, 32 * s, lane), vf[s], Y[r]);
      }
    }
    // Y fragments over tokens (accumulator k-order)
    bf16x8 yb[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) yb[s] = frag_from_acc(Y[2 * s], Y[2 * s + 1]);

    if constexpr (!OUT) {
      // segment maps, weights relative to the segment's end: token u = u0 + t of the chunk carries
      // g^{3L-1-u} = bq g^{63-t} (Q2) and g^{3L-2-2u} = bx g^{2(63-t)} (X1, X2)
      const int u0 = c * CP;
      const float bq = exp2f(a.log2g * (float)(3 * seglen - u0 - CP));
      const float bx = exp2f(a.log2g * (float)(3 * seglen - 2 * u0 - 2 * CP));
      bf16x8 qm[KC], zm[KC], yx[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        const bf16x8 qc = ld_cols(Qc, LDQ, 32 * s, 16 * mti, lane);
        const bf16x8 zc = w8_cols_sw(Zs, LDZ, 32 * s, 16 * mti, lane);
        f32x4 ylo, yhi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * s + kidx<bf16>(g, e);
          const float wx = bx * pw[2 * (CP - 1 - t)];
          qm[s][e] = (bf16)((float)qc[e] * (bq * pw[CP - 1 - t]));
          zm[s][e] = (bf16)((float)zc[e] * wx);
          if (e < 4) ylo[e] = Y[2 * s][e] * wx;
          else yhi[e - 4] = Y[2 * s + 1][e - 4] * wx;
        }
        yx[s] = frag_from_acc(ylo, yhi);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int s = 0; s < KC; ++s) {
          const bf16x8 qj = ld_cols(Qc, LDQ, 32 * s, 16 * (mtj0 + jj), lane);
          Q2m[jj] = mma(qm[s], qj, Q2m[jj]);
          X2m[jj] = mma(zm[s], qj, X2m[jj]);
        }
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int s = 0; s < KC; ++s) X1m[i] = mma(ld_cols(Qc, LDQ, 32 * s, 16 * i, lane), yx[s], X1m[i]);
    }
    // W <- g^192 W + Z~^T Y
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      f32x4 acc = W[i] * g192;
#pragma unroll
      for (int s = 0; s < KC; ++s) acc = mma(w8_cols_sw(Zts, LDT, 32 * s, 16 * i, lane), yb[s], acc);
      W[i] = acc;
    }

    __syncthreads();  // B2: Wm, the next chunk's rows and S0 visible

    // ======== phase 3: outputs, transposed (rows = the wave's value columns, columns = tau) ========
    // O^T = diag(g^{3(tau+1)}) W0^T Q^T + Y^T Wm^T, staged as rows
    if constexpr (OUT) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        f32x4 o = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) o = mma(w0b[s], w8_rows_acc(Qc, LDQ, 16 * r, 32 * s, lane), o);
        o *= of[r];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          if (32 * s <= 16 * r + 15) o = mma(yb[s], w8_rows_sw(Wms, LDW, 16 * r, 32 * s, lane), o);
        *(bf16x4 *)(Os + (16 * r + n) * LDO + vc0 + 4 * g) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
      }
    }
  }
  if constexpr (OUT) {
    if (nch > 0) {
      __syncthreads();  // the last chunk's staged rows
      flush_out(tok0 + (nch - 1) * CP);
    }
  }

  // ---------------- segment summary: S | P | W | Q2 | X1 | X2 ----------------
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * (a.nseg - 1) + seg) * SB;
    float *sQ2 = sb + PB, *sX1 = sQ2 + DK * DK, *sX2 = sX1 + DK * DV;
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sb[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n] = Sacc[i][j][r];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
        sb[DK * DK + o] = P[i][r];
        sb[DK * DK + DK * DV + o] = W[i][r];
        sX1[o] = X1m[i][r];
      }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * mti + 4 * g + r) * DK + 16 * (mtj0 + jj) + n;
        sQ2[o] = Q2m[jj][r];
        sX2[o] = X2m[jj][r];
      }
  }
  // ---------------- lead segment: its final state is the prefix of segment 1 ----------------
  if constexpr (OUT && LEAD) {
    float *pb = a.prefix + ((long)bh * a.nseg + seg + 1) * PB;
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n] = Sacc[i][j][r];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * i + 4 * g + r) * DV + vc0 + n;
        pb[DK * DK + o] = P[i][r];
        pb[DK * DK + DK * DV + o] = W[i][r];
      }
  }
}

// Walks segments (OUT ? seg_lo .. nseg-1 : 0 .. nseg-2) of every head, one workgroup each; one
// workgroup of eight waves per CU.
template <int DK, int DV, bool OUT>
__global__ void __launch_bounds__(512, 2) ho38_walk_kernel(Ho3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[H8Cfg<DK, DV, OUT>::BYTES];
  const int lo = OUT ? a.seg_lo : 0, nr = (OUT ? a.nseg : a.nseg - 1) - lo;
  ho38_body<DK, DV, OUT, false>(a, blockIdx.x / nr, lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head for its outputs and leave
// the prefix of segment 1; the rest summarise segments 1 .. nseg-2 of every head.  Both roles share
// one LDS allocation (the larger).
template <int DK, int DV>
__global__ void __launch_bounds__(512, 2) ho38_lead_kernel(Ho3Args a) {
  constexpr int BO = H8Cfg<DK, DV, true>::BYTES, BS = H8Cfg<DK, DV, false>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[BO > BS ? BO : BS];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    ho38_body<DK, DV, true, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = a.nseg - 2;
    ho38_body<DK, DV, false, false>(a, i / nr, 1 + i % nr, lds);
  }
}

hipError_t launch_ho38(int phase, int BH, const Ho3Args &a, hipStream_t s) {
  if (a.kc != 64) return hipErrorInvalidValue;
  switch (phase) {
    case HO3_SUMMARY:
      hipLaunchKernelGGL((ho38_walk_kernel<64, 128, false>), dim3(BH * (a.nseg - 1)), dim3(512), 0, s, a);
      return hipGetLastError();
    case HO3_OUTPUT:
      hipLaunchKernelGGL((ho38_walk_kernel<64, 128, true>), dim3(BH * (a.nseg - a.seg_lo)), dim3(512), 0, s, a);
      return hipGetLastError();
    case HO3_LEAD:
      if (a.nseg < 2 || a.nbh != BH) return hipErrorInvalidValue;
      hipLaunchKernelGGL((ho38_lead_kernel<64, 128>), dim3(BH * (a.nseg - 1)), dim3(512), 0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace hla2
