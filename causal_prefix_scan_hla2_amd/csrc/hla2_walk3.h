// hla2_walk3.h -- the bf16 chunk walker: one workgroup walks the 64-token
// chunks of one segment of one (b, h) sequence, carrying the corrected
// second-order state in fp32 accumulator registers.
//
// Method (technical summary of arXiv 2510.27258 on gist.science, §1 and §4),
// per token t with decay g:
//   S_t = g S_{t-1} + k_t k_t^T,  z_t = S_t q_t,
//   U_t = g^2 U_{t-1} + z_t v_t^T,  u_t = g^2 u_{t-1} + z_t,
//   num_t = q_t^T U_t,  den_t = q_t^T u_t,
// where U_t = S_t C_t - G_t and u_t = S_t m_t - h_t are the corrected
// products of the summary's output and normalisation formulas.  For a chunk
// (local index tau) entering with state (S0, U0, u0):
//   A   = Q K^T,  Ad[tau][i] = [i <= tau] g^{tau-i} A[tau][i]
//   Z   = diag(g^{tau+1}) Q S0 + Ad K                       (rows z_tau)
//   W   = [j <= tau] g^{2(tau-j)} (Q Z^T)[tau][j]
//   num = diag(g^{2(tau+1)}) Q U0 + W V,   den = diag(g^{2(tau+1)}) Q u0 + W 1
//   S  <- g^64 S0 + K^T diag(g^{63-t}) K
//   U  <- g^128 U0 + (diag(g^{2(63-t)}) Z)^T V,   u likewise with 1
// and in segment-summary mode also C <- g^64 C + Q^T diag(g^{63-t}) V and m
// likewise with 1.
//
// Work split (4 waves).  Wave w owns token block w (rows 16w..16w+15) for the
// chunk-local products A, Z and W, column tile(s) w of S, and the dv columns
// [DV/4 w, DV/4 (w+1)) of U, C, V and the output.  Each wave therefore keeps
// its V columns, its U columns (and their bf16 copy U0) and all of Q as MFMA
// operands in registers; only K, Q, V, Z, Z~ (the decayed Z), W and a bf16
// copy of S0 pass through LDS.  Products whose operand comes from an accumulator
// use the accumulator k-order of hla2_mfma.h (the other operand is read in that
// order too); products of two LDS operands read both as contiguous 16-byte
// vectors.  The output is produced transposed (out^T = U0^T Q^T + V^T W^T) so that
// each lane stores four consecutive values.
//
// Per chunk there are two workgroup barriers:
//   [A, Z, Z~ -> LDS; S update; C, m updates; operand fragments to registers]
//   B1
//   [S0 -> LDS; next chunk's K, Q, V -> LDS; W -> LDS; den; U, u updates]
//   B2
//   [outputs]
// The next chunk's global loads are issued at the top of a chunk and land in
// LDS after B1, so their latency overlaps phase 1.  Buffer loads return zero past the
// end of the sequence, so a ragged last chunk needs no special path: its zero
// rows add nothing to the outputs of its real rows, and the state after it is
// never used.
#pragma once
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

// Operand fragment in the contiguous k-order: lane (g, n) gets X[row0 + n][k0 + 8g + 0..7]
// with one 16-byte read.  Used for products whose two operands both come from LDS (both
// are read in this order).
__device__ __forceinline__ bf16x8 ld_rows_c(const bf16 *X, int ld, int row0, int k0, int lane) {
  return *(const bf16x8 *)(X + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// LDS byte address of an element, passed through an empty asm: reads made from different
// laundered addresses are never paired by the compiler into one (slower) paired read.
__device__ __forceinline__ unsigned lds_addr_opaque(const bf16 *p) {
  unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const bf16 *)p;
  asm("" : "+v"(a));
  return a;
}
__device__ __forceinline__ bf16x4 lds_ld4(unsigned a) {
  return *(__attribute__((address_space(3))) const bf16x4 *)(size_t)a;
}

// Column position of logical token j in a W row: within every 32 columns, the four
// 4-element groups a lane reads in the accumulator k-order (4g and 16 + 4g) sit side by
// side, so a fragment of W^T is one 16-byte read.
__device__ __forceinline__ int wpos(int j) {
  return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

template <int DK, int DV, bool OUT>
struct W3Cfg {
  static constexpr int CP = 64;            // tokens per chunk
  static constexpr int NB = CP / 16;       // token blocks
  static constexpr int NW = 4;             // waves, one token block each
  static constexpr int NT = 64 * NW;
  static constexpr int RT = DK / 16;       // 16-row tiles over d
  static constexpr int KD = DK / 32;       // k-steps over d
  static constexpr int KC = CP / 32;       // k-steps over chunk tokens
  static constexpr int SCT = RT / NW;      // S column tiles per wave
  static constexpr int UCT = DV / 16 / NW; // U / output column tiles per wave
  static constexpr int URT = RT / NW;      // row tiles of u (and m) per wave
  // Row pitches (elements) in LDS, chosen for how each buffer is read (gfx950 LDS:
  // 64 banks of 4 bytes).  Measured on the device: 16-byte reads of 16 rows at one
  // column and transpose reads of 8 rows x 32 bytes are conflict-free when rows start
  // 160 (or 288) bytes apart; 8-byte reads of 16 rows at one column are conflict-free
  // 144 bytes apart.  Two 8-byte reads that the compiler merges into one paired read
  // 32 bytes apart cost four times a plain read, so operands are read either as one
  // 16-byte vector per lane or as two separate 8-byte reads.
  static constexpr int LDK = DK + 16;      // K: 16-byte row reads and transpose reads
  static constexpr int LDQ = OUT ? DK + 8 : DK + 16;  // Q: 8-byte row reads (summary mode: transpose)
  static constexpr int LDT = DK + 16;      // Z~: transpose reads
  static constexpr int LDS0 = DK + 16;     // S0: 16-byte row reads
  static constexpr int LDZ = DK + 16;      // Z: 16-byte row reads
  static constexpr int LDV = DV + 16;      // V: transpose reads
  static constexpr int LDW = CP + 16;      // W: 16-byte row reads (columns permuted, see wpos)
  static constexpr int NVK = CP * DK / 8 / NT;  // 16-byte vectors per thread, Q and K
  static constexpr int NVV = CP * DV / 8 / NT;  // 16-byte vectors per thread, V
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + CP * LDQ;
  static constexpr int V_OFF = K_OFF + CP * LDK;
  static constexpr int ZT_OFF = V_OFF + CP * LDV;   // Z~ rows
  static constexpr int SB_OFF = ZT_OFF + CP * LDT;  // bf16 S0 rows
  static constexpr int Z_OFF = SB_OFF + DK * LDS0;  // Z rows   (output mode)
  static constexpr int W_OFF = Z_OFF + (OUT ? CP * LDZ : 0);  // W rows (output mode)
  static constexpr int ELEMS = W_OFF + (OUT ? CP * LDW : 0);
  static constexpr int LDS_BYTES = walk3_lds_bytes(DK, DV, OUT);
  static_assert(SCT >= 1 && UCT >= 1 && URT >= 1, "shape not supported by the 4-wave split");
  static_assert(NVK * NT * 8 == CP * DK && NVV * NT * 8 == CP * DV, "staging split");
  static_assert(ELEMS * 2 + (2 * CP + 1 + CP + 2 * DK) * 4 <= LDS_BYTES, "LDS accounting");
};

// LDS of one walker workgroup, carved from one byte array: the bf16 rows, u0 (double-
// buffered), the decay table and the chunk's den values.
template <int DK, int DV, bool OUT>
struct W3Lds {
  using Cfg = W3Cfg<DK, DV, OUT>;
  static constexpr int U0N = 2 * DK;  // u0s[2][DK]
  static constexpr int U0_OFF = Cfg::ELEMS * 2;
  static constexpr int PW_OFF = U0_OFF + U0N * 4;
  static constexpr int DENS_OFF = PW_OFF + (2 * Cfg::CP + 1) * 4;
  static constexpr int BYTES = DENS_OFF + Cfg::CP * 4;
  static_assert(U0_OFF % 16 == 0, "u0 rows are read as 16-byte vectors");
  static_assert(BYTES <= Cfg::LDS_BYTES, "LDS accounting");
};

// One workgroup's walk of segment `seg` of head `bh`.  With LEAD (output mode, segment 0 of
// a plan with more than one segment) the state after the segment is written, in fp32, as
// the prefix block of segment 1, so that no summary of segment 0 is needed.
template <int DK, int DV, bool OUT, bool DEC, bool DEN, bool LEAD>
__device__ __forceinline__ void walk3_body(const WalkArgs &a, const int bh, const int seg, unsigned char *lds) {
  using Cfg = W3Cfg<DK, DV, OUT>;
  using L = W3Lds<DK, DV, OUT>;
  constexpr int CP = Cfg::CP, NB = Cfg::NB, NT = Cfg::NT, RT = Cfg::RT, KD = Cfg::KD, KC = Cfg::KC;
  constexpr int SCT = Cfg::SCT, UCT = Cfg::UCT, URT = Cfg::URT;
  constexpr bool PAIR = UCT == 2 && DK == 64;  // interleaved value-column tiles (see vcol)
  constexpr int LDK = Cfg::LDK, LDQ = Cfg::LDQ, LDT = Cfg::LDT, LDS0 = Cfg::LDS0, LDZ = Cfg::LDZ;
  constexpr int LDV = Cfg::LDV, LDW = Cfg::LDW, NVK = Cfg::NVK, NVV = Cfg::NVV;

  bf16 *const smem = (bf16 *)lds;
  float *const pw = (float *)(lds + L::PW_OFF);      // decay^x, x = 0 .. 2 CP
  float *const dens = (float *)(lds + L::DENS_OFF);  // den of the chunk's rows
  float(*const u0s)[DK] = (float(*)[DK])(lds + L::U0_OFF);  // u0, double-buffered
  bf16 *const Qs = smem + Cfg::Q_OFF;
  bf16 *const Ks = smem + Cfg::K_OFF;
  bf16 *const Vs = smem + Cfg::V_OFF;
  bf16 *const Zts = smem + Cfg::ZT_OFF;
  bf16 *const Sb = smem + Cfg::SB_OFF;
  bf16 *const Zs = smem + Cfg::Z_OFF;
  bf16 *const Ws = smem + Cfg::W_OFF;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Value column of lane n in the wave's column tile j (of U, C, V and the outputs).  With two
  // tiles per wave at d <= 64 the tiles interleave in 4-column groups, so that a lane's outputs
  // of both tiles are 8 consecutive columns (one 16-byte store); V is stored in LDS with the
  // matching permutation so that its column fragments stay plain transpose reads.  (Measured:
  // the d = 128 walker, one wave per SIMD, is slower with it.)
  auto vcol = [&](int j, int nn) __attribute__((always_inline)) -> int {
    if constexpr (PAIR) return 32 * w + 8 * (nn >> 2) + 4 * j + (nn & 3);
    return 16 * (w * UCT + j) + nn;
  };
  const int d = a.d, dv = a.dv;
  const int tok0 = walk_seg_chunk0(a, seg) * CP;  // first token of the segment
  const int tokE = min(a.n, tok0 + walk_seg_chunks(a, seg) * CP);
  // a summary of the last segment (final state) stops at its last full chunk
  const int nch = (!OUT && seg == a.nseg - 1) ? (tokE - tok0) / CP : (tokE - tok0 + CP - 1) / CP;

  // buffer resources over this head's rows; reads past the end return zero
  const long hq = (long)bh * a.n * d, hv = (long)bh * a.n * dv;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc((const bf16 *)a.q + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc((const bf16 *)a.k + hq, a.n * d * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc((const bf16 *)a.v + hv, a.n * dv * 2);
  const __amdgpu_buffer_rsrc_t ro = buf_rsrc((bf16 *)a.out + hv, OUT ? a.n * dv * 2 : 0);
  // den_out may be null: then the resource covers no bytes (over a valid base) and every
  // store is dropped
  const __amdgpu_buffer_rsrc_t rden_out = buf_rsrc(
      a.den_out ? (const void *)(a.den_out + (long)bh * a.n) : a.q, (OUT && a.den_out) ? a.n * 4 : 0);

  for (int x = tid; x <= 2 * CP; x += NT) pw[x] = DEC ? exp2f((float)x * a.log2g) : 1.0f;

  // ---------------- staging of one chunk: global -> registers -> LDS ----------------
  u32x4 rgq[NVK], rgk[NVK], rgv[NVV];
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const int t0 = tok0 + c * CP;
    // padded columns (e0 >= d) read at an offset past the buffer, which returns zero, so
    // no select waits on the data
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
  auto store_chunk = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NVK; ++i) {
      const int vi = tid + i * NT, t = vi / (DK / 8), e0 = 8 * (vi % (DK / 8));
      *(u32x4 *)(Qs + t * LDQ + e0) = rgq[i];
      *(u32x4 *)(Ks + t * LDK + e0) = rgk[i];
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int vi = tid + i * NT, t = vi / (DV / 8), e0 = 8 * (vi % (DV / 8));
      if constexpr (PAIR) {
        // value columns 8a + 4j + b of each 32 are stored at 16j + 4a + b (see vcol)
        const int base = (e0 & ~31) + 4 * ((e0 & 31) >> 3);
        *(u32x2 *)(Vs + t * LDV + base) = u32x2{rgv[i][0], rgv[i][1]};
        *(u32x2 *)(Vs + t * LDV + base + 16) = u32x2{rgv[i][2], rgv[i][3]};
      } else {
        *(u32x4 *)(Vs + t * LDV + e0) = rgv[i];
      }
    }
  };

  // ---------------- state ----------------
  f32x4 Sacc[RT][SCT], Uacc[RT][UCT], uacc[URT];
  f32x4 Cacc[OUT ? 1 : RT][OUT ? 1 : UCT], macc[OUT ? 1 : URT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
#pragma unroll
    for (int j = 0; j < SCT; ++j) Sacc[i][j] = zero4();
#pragma unroll
    for (int j = 0; j < UCT; ++j) Uacc[i][j] = zero4();
    if constexpr (!OUT) {
#pragma unroll
      for (int j = 0; j < UCT; ++j) Cacc[i][j] = zero4();
    }
  }
#pragma unroll
  for (int r = 0; r < URT; ++r) {
    uacc[r] = zero4();
    if constexpr (!OUT) macc[r] = zero4();
  }
  if (OUT && seg > 0) {
    const float *pb = a.prefix + ((long)bh * a.nseg + seg) * prefix_block_floats(DK, DV);
    const float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[i][j][r] = pS[(16 * i + 4 * g + r) * DK + 16 * (w * SCT + j) + n];
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Uacc[i][j][r] = pU[(16 * i + 4 * g + r) * DV + vcol(j, n)];
    }
    if constexpr (DEN) {
#pragma unroll
      for (int ur = 0; ur < URT; ++ur)
#pragma unroll
        for (int r = 0; r < 4; ++r) uacc[ur][r] = n == 0 ? pu[16 * (w * URT + ur) + 4 * g + r] : 0.f;
    }
  }
  // S0 as bf16 rows (S is symmetric: the wave's column tile written as rows)
  auto write_S0 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j) st4(Sb + (16 * (w * SCT + j) + n) * LDS0 + 16 * i + 4 * g, Sacc[i][j]);
  };
  auto write_u0 = [&](int buf) __attribute__((always_inline)) {
    if constexpr (DEN) {
      if (n == 0) {
#pragma unroll
        for (int ur = 0; ur < URT; ++ur) *(f32x4 *)(&u0s[buf][16 * (w * URT + ur) + 4 * g]) = uacc[ur];
      }
    }
  };

  // ---------------- loop-invariant factors ----------------
  __syncthreads();  // pw
  const int tau_w = 16 * w + n;  // this lane's row in the wave's token block
  // Aᵀ / Wᵀ tile I of the wave's block: element r is (i = 16 I + 4 g + r, tau = tau_w).
  // Off-diagonal tiles (I < w) use g^{16(w-I-1)} * g^{16 + n - 4g - r}; the diagonal tile
  // masks i > tau.  All exponents are >= 0.
  float fa_off[4], fa_dg[4], kfh[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = n - 4 * g - r;
    fa_off[r] = DEC ? pw[16 + e] : 1.f;
    const int ep = e >= 0 ? e : 0;
    fa_dg[r] = e >= 0 ? (DEC ? pw[ep] : 1.f) : 0.f;
    kfh[r] = DEC ? pw[15 - 4 * g - r] : 1.f;  // token weights g^{63-t}: see kweight()
  }
  const float zf = DEC ? pw[tau_w + 1] : 1.f;            // g^{tau+1}
  const float ztf = DEC ? pw[2 * (CP - 1 - tau_w)] : 1.f;  // g^{2(63-tau)}
  const float g64 = DEC ? pw[CP] : 1.f, g128 = DEC ? pw[2 * CP] : 1.f;
  // weight g^{63-t} of token t = 32 s + kidx(g, e) in a k-step fragment
  auto kweight = [&](int s, int e) __attribute__((always_inline)) -> float {
    // e < 4: t = 32 s + 4 g + e;  e >= 4: t = 32 s + 16 + 4 g + (e - 4)
    // 63 - t = (48 - 32 s) + (15 - 4 g - e)  or  (32 - 32 s) + (15 - 4 g - (e - 4))
    if (!DEC) return 1.f;
    return e < 4 ? pw[48 - 32 * s] * kfh[e] : pw[32 - 32 * s] * kfh[e - 4];
  };
  // ones column (u, m): B fragment with 1 (or the token weight) in column 0
  bf16x8 ones, onesw[KC];
  {
    const bf16 o = (bf16)(n == 0 ? 1.f : 0.f);
    ones = bf16x8{o, o, o, o, o, o, o, o};
#pragma unroll
    for (int s = 0; s < KC; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) onesw[s][e] = (bf16)(n == 0 ? kweight(s, e) : 0.f);
  }

  // ---------------- prologue ----------------
  load_chunk(0);
  write_S0();
  write_u0(0);
  store_chunk();
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    // the next chunk's loads fly during phase 1 and land in LDS after B1
    // (a repeat of the last chunk at the end; it is never read)
    load_chunk(min(c + 1, nch - 1));
    // keep the loads here: left to itself the scheduler sinks them to just before B1 and
    // waits on them at once, exposing the whole memory latency every chunk.  (Measured:
    // the d = 128 output walk, one wave per SIMD and at its register limit, runs faster
    // with the scheduler's placement.)
    if constexpr (!(OUT && DK > 64)) __builtin_amdgcn_sched_barrier(0);

    // ======== phase 1: chunk-local products of the wave's token block ========
    bf16x8 qw[KD];
#pragma unroll
    for (int s = 0; s < KD; ++s) qw[s] = ld_rows_c(Qs, LDQ, 16 * w, 32 * s, lane);

    // A^T tiles (rows i, column tau of the block) -> masked, decayed -> Ad^T fragments.
    // Every wave computes all tiles and zeroes those above its block: the products
    // never sit under a branch (the waves with later blocks bound the time anyway).
    bf16x8 adf[KC];
    {
      f32x4 at[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        at[I] = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) at[I] = mma(ld_rows_c(Ks, LDK, 16 * I, 32 * s, lane), qw[s], at[I]);
        const float sc = DEC ? pw[16 * max(w - I - 1, 0)] : 1.f;  // uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) at[I][r] *= I < w ? sc * fa_off[r] : (I == w ? fa_dg[r] : 0.f);
      }
#pragma unroll
      for (int s = 0; s < KC; ++s) adf[s] = frag_from_acc(at[2 * s], at[2 * s + 1]);
    }

    // token-weighted K columns of the wave's S column tiles (B operand of the S update)
    bf16x8 kb[SCT][KC];
#pragma unroll
    for (int j = 0; j < SCT; ++j)
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        kb[j][s] = ld_cols(Ks, LDK, 32 * s, 16 * (w * SCT + j), lane);
        if (DEC) {
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[j][s][e] = (bf16)((float)kb[j][s][e] * kweight(s, e));
        }
      }

    // per 16-row tile i of d, with the K^T fragments of that tile (A operand, k = tokens):
    //   Z^T tile (rows d, column tau): S0 Q_w^T scaled by g^{tau+1}, plus K^T Ad_w^T;
    //   S <- g^64 S + K^T diag(g^{63-t}) K on the wave's column tiles.
    // One row tile at a time keeps few K^T fragments live.
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      bf16x8 kt[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) kt[s] = ld_cols(Ks, LDK, 32 * s, 16 * i, lane);
      f32x4 z = zero4();
#pragma unroll
      for (int s = 0; s < KD; ++s) z = mma(ld_rows_c(Sb, LDS0, 16 * i, 32 * s, lane), qw[s], z);
      if (DEC) z *= zf;
#pragma unroll
      for (int s = 0; s < KC; ++s) z = mma(kt[s], adf[s], z);
      // Z[tau][16 i + 4 g + r] and its decayed copy, as rows
      if constexpr (OUT) st4(Zs + tau_w * LDZ + 16 * i + 4 * g, z);
      st4(Zts + tau_w * LDT + 16 * i + 4 * g, DEC ? z * ztf : z);
#pragma unroll
      for (int j = 0; j < SCT; ++j) {
        f32x4 acc = DEC ? Sacc[i][j] * g64 : Sacc[i][j];
#pragma unroll
        for (int s = 0; s < KC; ++s) acc = mma(kt[s], kb[j][s], acc);
        Sacc[i][j] = acc;
      }
    }

    // V column fragments of the wave (B operand of the U update, A operand of out^T)
    bf16x8 vf[UCT][KC];
#pragma unroll
    for (int j = 0; j < UCT; ++j)
#pragma unroll
      for (int s = 0; s < KC; ++s) vf[j][s] = ld_cols(Vs, LDV, 32 * s, 16 * (w * UCT + j), lane);

    // Q fragments of every row tile (B operand of out^T), in the accumulator k-order of U0:
    // two separate 8-byte reads per fragment, from one opaque base per (k-step, half)
    bf16x8 qall[OUT ? NB : 1][KD];
    if constexpr (OUT) {
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        const unsigned a0 = lds_addr_opaque(Qs + n * LDQ + 32 * s + 4 * g);
        const unsigned a1 = lds_addr_opaque(Qs + n * LDQ + 32 * s + 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < NB; ++r)
          qall[r][s] = cat8(lds_ld4(a0 + 2 * 16 * r * LDQ), lds_ld4(a1 + 2 * 16 * r * LDQ));
      }
    }

    if constexpr (!OUT) {
      // C <- g^64 C + Q^T diag(g^{63-t}) V, m likewise with the weighted ones column;
      // one row tile of Q^T fragments at a time
      bf16x8 vb[UCT][KC];
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int s = 0; s < KC; ++s) {
          vb[j][s] = vf[j][s];
          if (DEC) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vb[j][s][e] = (bf16)((float)vb[j][s][e] * kweight(s, e));
          }
        }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        bf16x8 qt[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s) qt[s] = ld_cols(Qs, LDQ, 32 * s, 16 * i, lane);
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 acc = DEC ? Cacc[i][j] * g64 : Cacc[i][j];
#pragma unroll
          for (int s = 0; s < KC; ++s) acc = mma(qt[s], vb[j][s], acc);
          Cacc[i][j] = acc;
        }
      }
      if constexpr (DEN) {
#pragma unroll
        for (int ur = 0; ur < URT; ++ur) {
          f32x4 acc = DEC ? macc[ur] * g64 : macc[ur];
#pragma unroll
          for (int s = 0; s < KC; ++s) acc = mma(ld_cols(Qs, LDQ, 32 * s, 16 * (w * URT + ur), lane), onesw[s], acc);
          macc[ur] = acc;
        }
      }
    }

    // bf16 U0 columns of the wave (A operand of out^T), taken before the U update
    bf16x8 u0b[OUT ? UCT : 1][KD];
    if constexpr (OUT) {
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int s = 0; s < KD; ++s) u0b[j][s] = frag_from_acc(Uacc[2 * s][j], Uacc[2 * s + 1][j]);
    }

    __syncthreads();  // B1: Z, Z~ visible; every read of this chunk's Q, K, V, S0 is done

    // ======== phase 2 ========
    write_S0();
    store_chunk();

    if constexpr (OUT) {
      // W^T tiles J <= w (rows j, column tau) -> masked, decayed -> W rows in LDS; den
      float rs = 0.f;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        f32x4 wt = zero4();
#pragma unroll
        for (int s = 0; s < KD; ++s) wt = mma(ld_rows_c(Zs, LDZ, 16 * J, 32 * s, lane), qw[s], wt);
        const float sc = DEC ? pw[32 * max(w - J - 1, 0)] : 1.f;  // uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // the W factors are the squares of the A factors; squared here rather than kept
          // in registers across the chunk loop
          float fo = fa_off[r], fd = fa_dg[r];
          asm volatile("" : "+v"(fo), "+v"(fd));
          wt[r] *= J < w ? sc * (fo * fo) : (J == w ? fd * fd : 0.f);
        }
        if constexpr (DEN) rs += (wt[0] + wt[1]) + (wt[2] + wt[3]);
        st4(Ws + tau_w * LDW + wpos(16 * J + 4 * g), wt);
      }
      if constexpr (DEN) {
        // den_tau = g^{2(tau+1)} q_tau . u0 + sum_j W[tau][j]
        const float *u0 = u0s[c & 1];
        float qu = 0.f;
#pragma unroll
        for (int s = 0; s < KD; ++s) {  // qw holds k = 32 s + 8 g + 0..7
          const f32x4 ua = *(const f32x4 *)(u0 + 32 * s + 8 * g);
          const f32x4 ub = *(const f32x4 *)(u0 + 32 * s + 8 * g + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) qu += (float)qw[s][e] * ua[e] + (float)qw[s][4 + e] * ub[e];
        }
        qu = sum_groups(qu);
        rs = sum_groups(rs);
        const float den = (DEC ? pw[2 * (tau_w + 1)] : 1.f) * qu + rs;
        if (g == 0) dens[tau_w] = den;
        // den_t to the caller's buffer; rows past the end fall outside the buffer and are dropped
        const int t = tok0 + c * CP + tau_w;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, den), rden_out,
                                              g == 0 ? t * 4 : 0x7fffffff, 0, 0);
      }
    }

    // U <- g^128 U + Z~^T V (the wave's columns); u likewise with the ones column
    {
      bf16x8 zt[RT][KC];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int s = 0; s < KC; ++s) zt[i][s] = ld_cols(Zts, LDT, 32 * s, 16 * i, lane);
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 acc = DEC ? Uacc[i][j] * g128 : Uacc[i][j];
#pragma unroll
          for (int s = 0; s < KC; ++s) acc = mma(zt[i][s], vf[j][s], acc);
          Uacc[i][j] = acc;
        }
      if constexpr (DEN) {
#pragma unroll
        for (int ur = 0; ur < URT; ++ur) {
          f32x4 acc = DEC ? uacc[ur] * g128 : uacc[ur];
#pragma unroll
          for (int s = 0; s < KC; ++s) acc = mma(ld_cols(Zts, LDT, 32 * s, 16 * (w * URT + ur), lane), ones, acc);
          uacc[ur] = acc;
        }
        if constexpr (OUT) write_u0((c + 1) & 1);
      }
    }

    __syncthreads();  // B2: W, den, the next chunk's Q, K, V and S0 visible

    // ======== phase 3: outputs (transposed tiles: rows = value columns, columns = tau) ========
    if constexpr (OUT) {
      const int t0 = tok0 + c * CP;
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        const float of = DEC ? pw[2 * (16 * r + n + 1)] : 1.f;
        float rden = 1.f;
        if constexpr (DEN) {
          if (a.normalize) rden = 1.f / dens[16 * r + n];
        }
        bf16x8 wb[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          if (32 * s <= 16 * r + 15) wb[s] = ld_rows_c(Ws, LDW, 16 * r, 32 * s, lane);
        bf16x4 ob[UCT];
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 o = zero4();
#pragma unroll
          for (int s = 0; s < KD; ++s) o = mma(u0b[j][s], qall[r][s], o);
          if (DEC) o *= of;
#pragma unroll
          for (int s = 0; s < KC; ++s)
            if (32 * s <= 16 * r + 15) o = mma(vf[j][s], wb[s], o);
          if (DEN) o *= rden;
          ob[j] = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        }
        // rows past the end fall outside the buffer; padded columns are sent there too
        const int t = t0 + 16 * r + n;
        if constexpr (PAIR) {
          const int col = vcol(0, 4 * g);  // 8 consecutive columns: tile 0's four, then tile 1's
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, cat8(ob[0], ob[1])), ro,
                                                 col < dv ? (t * dv + col) * 2 : 0x7fffffff, 0, 0);
        } else {
#pragma unroll
          for (int j = 0; j < UCT; ++j) {
            const int col = vcol(j, 4 * g);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob[j]), ro,
                                                  col < dv ? (t * dv + col) * 2 : 0x7fffffff, 0, 0);
          }
        }
      }
    }
  }

  // ---------------- segment summary: S | C | U | m | u ----------------
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * walk_nsum(a) + seg) * sum_block_floats(DK, DV);
    float *sS = sb, *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(16 * i + 4 * g + r) * DK + 16 * (w * SCT + j) + n] = Sacc[i][j][r];
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sC[(16 * i + 4 * g + r) * DV + vcol(j, n)] = Cacc[i][j][r];
          sU[(16 * i + 4 * g + r) * DV + vcol(j, n)] = Uacc[i][j][r];
        }
    }
    if (n == 0) {
#pragma unroll
      for (int ur = 0; ur < URT; ++ur) {
        const int row = 16 * (w * URT + ur) + 4 * g;
        *(f32x4 *)(sm + row) = DEN ? macc[ur] : zero4();
        *(f32x4 *)(su + row) = DEN ? uacc[ur] : zero4();
      }
    }
  }

  // ---------------- lead segment: its final state is the prefix S0 | U0 | u0 of segment 1 ----------------
  // (the layout the prefix is read in above; u0 is zero when den is not carried)
  if constexpr (OUT && LEAD) {
    float *pb = a.prefix_out + ((long)bh * a.nseg + seg + 1) * prefix_block_floats(DK, DV);
    float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) pS[(16 * i + 4 * g + r) * DK + 16 * (w * SCT + j) + n] = Sacc[i][j][r];
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) pU[(16 * i + 4 * g + r) * DV + vcol(j, n)] = Uacc[i][j][r];
    }
    if (n == 0) {
#pragma unroll
      for (int ur = 0; ur < URT; ++ur) *(f32x4 *)(pu + 16 * (w * URT + ur) + 4 * g) = DEN ? uacc[ur] : zero4();
    }
  }
}

// Walks segments seg_lo .. (nseg or nsum) - 1 of every head, one workgroup each.
template <int DK, int DV, bool OUT, bool DEC, bool DEN>
__global__ void __launch_bounds__(256, (walk3_waves_per_eu(DK, DV, OUT)))
walk3_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[W3Lds<DK, DV, OUT>::BYTES];
  const int nr = (OUT ? a.nseg : walk_nsum(a)) - a.seg_lo;  // segments of a head in this launch
  walk3_body<DK, DV, OUT, DEC, DEN, false>(a, blockIdx.x / nr, a.seg_lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head in output mode and
// leave the prefix of segment 1; the rest summarise segments 1 .. nsum-1 of every head.
// Both roles share one LDS allocation (the larger, output mode's), so the launch holds as
// many workgroups per CU as the output walk.
template <int DK, int DV, bool DEC, bool DEN>
__global__ void __launch_bounds__(256, (walk3_waves_per_eu(DK, DV, true)))
walk3_lead_kernel(WalkArgs a) {
  constexpr int BO = W3Lds<DK, DV, true>::BYTES, BS = W3Lds<DK, DV, false>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[BO > BS ? BO : BS];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    walk3_body<DK, DV, true, DEC, DEN, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = walk_nsum(a) - 1;
    walk3_body<DK, DV, false, DEC, DEN, false>(a, i / nr, 1 + i % nr, lds);
  }
}

template <int DK, int DV>
hipError_t launch_walk3_t(bool out, bool dec, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
#define HLA2_W3(O, D, N)                                                                     \
  if (out == O && dec == D && den == N) {                                                    \
    hipLaunchKernelGGL((walk3_kernel<DK, DV, O, D, N>), grid, dim3(256), 0, s, a);          \
    return hipGetLastError();                                                                \
  }
  HLA2_W3(true, true, true)
  HLA2_W3(true, true, false)
  HLA2_W3(true, false, true)
  HLA2_W3(true, false, false)
  HLA2_W3(false, true, true)
  HLA2_W3(false, true, false)
  HLA2_W3(false, false, true)
  HLA2_W3(false, false, false)
#undef HLA2_W3
  return hipErrorInvalidValue;
}

template <int DK, int DV>
hipError_t launch_walk3_lead_t(bool dec, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
#define HLA2_W3L(D, N)                                                                       \
  if (dec == D && den == N) {                                                                \
    hipLaunchKernelGGL((walk3_lead_kernel<DK, DV, D, N>), grid, dim3(256), 0, s, a);        \
    return hipGetLastError();                                                                \
  }
  HLA2_W3L(true, true)
  HLA2_W3L(true, false)
  HLA2_W3L(false, true)
  HLA2_W3L(false, false)
#undef HLA2_W3L
  return hipErrorInvalidValue;
}

}  // namespace hla2
