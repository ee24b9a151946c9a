// hla2_walk8.h -- the bf16 chunk walker with eight waves: one workgroup walks the 64-token
// chunks of one segment of one (b, h) sequence, carrying the corrected second-order state in
// fp32 accumulator registers.
//
// Method (technical summary of arXiv 2510.27258 on gist.science, §1 and §4), per token t with
// decay g:
//   S_t = g S_{t-1} + k_t k_t^T,  z_t = S_t q_t,
//   U_t = g^2 U_{t-1} + z_t v_t^T,  u_t = g^2 u_{t-1} + z_t,
//   num_t = q_t^T U_t,  den_t = q_t^T u_t,
// where U_t = S_t C_t - G_t and u_t = S_t m_t - h_t are the corrected products of the
// summary's output and normalisation formulas.  For a chunk (local index tau) entering with
// state (S0, U0, u0):
//   A   = Q K^T,  Ad[tau][i] = [i <= tau] g^{tau-i} A[tau][i]
//   Z   = diag(g^{tau+1}) Q S0 + Ad K                       (rows z_tau)
//   W   = [j <= tau] g^{2(tau-j)} (Q Z^T)[tau][j]
//   num = diag(g^{2(tau+1)}) Q U0 + W V,   den = diag(g^{2(tau+1)}) Q u0 + W 1
//   S  <- g^64 S0 + K^T diag(g^{63-t}) K
//   U  <- g^128 U0 + (diag(g^{2(63-t)}) Z)^T V,   u likewise with 1
// and in segment-summary mode also C <- g^64 C + Q^T diag(g^{63-t}) V and m likewise with 1.
//
// Work split.  Eight waves put two on every SIMD of the CU, so that one wave's dependency
// chain (an MFMA result scaled on the VALU, converted, passed through LDS) overlaps the other
// wave's.  Wave w = 4 h + b works on token block b (rows 16b .. 16b+15) and half h:
//   - the chunk-local tiles of its block: A^T (all four, in both halves), Z^T of d-row tiles
//     [h RT/2, (h+1) RT/2), and W^T of column tiles {2h, 2h+1};
//   - the S tiles in those d-row tiles and in column tiles [b RT/4, (b+1) RT/4);
//   - at dv = 128 the value column tile w of U (C), V and the output for all four token
//     blocks; at dv = 64 the value column tile b of U (both halves carry it) and the outputs
//     of token blocks {2h, 2h+1}.
// Its U columns, the bf16 copy U0 and its V columns are MFMA operands in registers; K, Q (two
// buffers, so the output phase still reads this chunk's Q after the next one is staged), V,
// Z, Z~ (the decayed Z), W and a bf16 copy of S0 pass through LDS.  Products whose operand
// comes from an accumulator use the accumulator k-order of hla2_mfma.h; products of two LDS
// operands read both as contiguous 16-byte vectors.  The output is produced transposed
// (out^T = U0^T Q^T + V^T W^T) so that each lane stores four consecutive values.
//
// Per chunk there are two workgroup barriers:
//   [A, Z, Z~ -> LDS; S update; C, m updates; operand fragments to registers]
//   B1
//   [S0 -> LDS; W -> LDS; den parts; next chunk's K, Q, V -> LDS; U, u updates]
//   (the next chunk's rows go in before W except at d = 64, dv = 128)
//   B2
//   [outputs]
// The next chunk's global loads are issued at the top of a chunk and land in LDS after B1, so
// their latency overlaps phase 1.  Buffer loads return zero past the end of the sequence, so a
// ragged last chunk needs no special path: its zero rows add nothing to the outputs of its real
// rows, and the state after it is never used.  No MFMA sits under a runtime branch: every
// per-wave difference is an address or a factor.
#pragma once
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

// Operand fragment in the contiguous k-order: lane (g, n) gets X[row0 + n][k0 + 8g + 0..7]
// with one 16-byte read.  Used for products whose two operands both come from LDS (both
// are read in this order).
__device__ __forceinline__ bf16x8 w8_rows(const bf16 *X, int ld, int row0, int k0, int lane) {
  return *(const bf16x8 *)(X + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// Swizzled rows.  The buffers that take 8-byte row writes from accumulator tiles (lane (g, n)
// writes row n) keep the 16-byte piece j of row r at piece j ^ ((r >> 2) & 1).  Measured on the
// device at a 160-byte pitch (cycles of LDS time per wave-wide access): 8-byte accumulator-row
// writes 16 -> 8, while 16-byte row reads stay at 4 and transpose reads of 8 rows at 2 (a swizzle
// on row bit 3 instead also halves the writes but doubles the 16-byte reads).  In elements: column
// c of row r sits at c ^ (((r >> 2) & 1) << 3).

// The swizzle of a lane's row in an accumulator-row access (row 16 x + n): bit 2 of n.  Column
// bases that are multiples of 16 keep bit 3 clear, so the swizzled column is base + (lane part ^
// sw) and the base stays a constant offset of the access.
__device__ __forceinline__ int w8_swl(int lane) { return ((lane >> 2) & 1) << 3; }

// w8_rows on a swizzled buffer (row0 and k0 multiples of 16)
__device__ __forceinline__ bf16x8 w8_rows_sw(const bf16 *X, int ld, int row0, int k0, int lane) {
  return *(const bf16x8 *)(X + (row0 + (lane & 15)) * ld + k0 + ((8 * (lane >> 4)) ^ w8_swl(lane)));
}

// ld_cols on a swizzled buffer (k0 a multiple of 32, col0 of 16): lane (g, n) gets
// X[k-order of group g][col0 + n]; its rows k0 + 4 g + 0..3 (and 16 further) have bit 2 = g & 1
__device__ __forceinline__ bf16x8 w8_cols_sw(const bf16 *X, int ld, int k0, int col0, int lane) {
  const int g = lane >> 4, src = lane & 15;
  const bf16 *p = X + (k0 + 4 * g + (src >> 2)) * ld + col0 + ((4 * (src & 3)) ^ ((g & 1) << 3));
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * ld));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}

// LDS byte address of an element, passed through an empty asm: reads made from different
// laundered addresses are never paired by the compiler into one (slower) paired read.
__device__ __forceinline__ unsigned w8_lds_addr(const bf16 *p) {
  unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const bf16 *)p;
  asm("" : "+v"(a));
  return a;
}
__device__ __forceinline__ bf16x4 w8_ld4(unsigned a) {
  return *(__attribute__((address_space(3))) const bf16x4 *)(size_t)a;
}

// Row fragment in the accumulator k-order: lane (g, n) gets X[row0 + n][k0 + 4g + 0..3,
// k0 + 16 + 4g + 0..3] with two 8-byte reads, each from its own opaque base.
__device__ __forceinline__ bf16x8 w8_rows_acc(const bf16 *X, int ld, int row0, int k0, int lane) {
  const bf16 *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  return cat8(w8_ld4(w8_lds_addr(p)), w8_ld4(w8_lds_addr(p + 16)));
}

// Column position of logical token j in a W row: within every 32 columns, the four 4-element
// groups a lane reads in the accumulator k-order (4g and 16 + 4g) sit side by side, so a
// fragment of W^T is one 16-byte read.
__device__ __forceinline__ int w8_wpos(int j) {
  return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

template <int DK, int DV, bool OUT>
struct W8Cfg {
  static constexpr int CP = 64;             // tokens per chunk
  static constexpr int NB = CP / 16;        // token blocks
  static constexpr int NW = 8;              // waves: block w % 4, half w / 4
  static constexpr int NT = 64 * NW;
  static constexpr int RT = DK / 16;        // 16-row tiles over d
  static constexpr int KD = DK / 32;        // k-steps over d
  static constexpr int KC = CP / 32;        // k-steps over chunk tokens
  static constexpr int CT = DV / 16;        // value column tiles
  static constexpr bool VSPLIT = CT >= NW;  // every wave owns CT / 8 value column tiles
  static constexpr int UCT = VSPLIT ? CT / NW : 1;   // value column tiles per wave
  static constexpr int NBO = VSPLIT ? NB : NB / 2;   // output token blocks per wave
  static constexpr int SCT = RT / 4;        // S column tiles per wave
  static constexpr int SRT = RT / 2;        // S (and Z^T) d-row tiles per wave
  static constexpr int NQB = OUT ? 2 : 1;   // Q buffers
  // Outputs staged as rows in LDS and stored as contiguous 16-byte pieces (d <= 64; at d = 128
  // there is no room, and each lane stores its four values of a row from registers)
  static constexpr bool OST = OUT && DK <= 64;
  static constexpr int LDO = DV + 8;       // staged output rows: 8-byte writes, 16-byte reads
  // Row pitches (elements) in LDS, chosen for how each buffer is read (gfx950 LDS: 64 banks of
  // 4 bytes).  Measured on the device: 16-byte reads of 16 rows at one column and transpose
  // reads of 8 rows x 32 bytes are conflict-free when rows start 160 (or 288) bytes apart;
  // 8-byte reads of 16 rows at one column are conflict-free 144 bytes apart.  Z~, S0, Z and W,
  // which also take 8-byte row writes, are swizzled (w8_sw).
  static constexpr int LDK = DK + 16;      // K: 16-byte row reads and transpose reads
  static constexpr int LDQ = OUT ? DK + 8 : DK + 16;  // Q: 8-byte row reads (summary mode: transpose)
  static constexpr int LDT = DK + 16;      // Z~: transpose reads
  static constexpr int LDS0 = DK + 16;     // S0: 16-byte row reads
  static constexpr int LDZ = DK + 16;      // Z: 16-byte row reads
  static constexpr int LDV = DV + 16;      // V: transpose reads
  static constexpr int LDW = CP + 16;      // W: 16-byte row reads (columns permuted, see w8_wpos)
  static constexpr int NVK = CP * DK / 8 / NT;  // 16-byte vectors per thread, Q and K
  static constexpr int NVV = CP * DV / 8 / NT;  // 16-byte vectors per thread, V
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + NQB * CP * LDQ;
  static constexpr int V_OFF = K_OFF + CP * LDK;
  static constexpr int ZT_OFF = V_OFF + CP * LDV;   // Z~ rows
  static constexpr int SB_OFF = ZT_OFF + CP * LDT;  // bf16 S0 rows
  static constexpr int Z_OFF = SB_OFF + DK * LDS0;  // Z rows   (output mode)
  static constexpr int W_OFF = Z_OFF + (OUT ? CP * LDZ : 0);  // W rows (output mode)
  static constexpr int O_OFF = W_OFF + (OUT ? CP * LDW : 0);   // staged output rows (OST)
  static constexpr int ELEMS = O_OFF + (OST ? CP * LDO : 0);
  static constexpr int NPO = CP * DV / 8 / NT;  // 16-byte output pieces per thread (OST)
  static_assert(SCT >= 1 && SRT >= 1 && NVK >= 1 && NVV >= 1, "shape not supported by the 8-wave split");
  static_assert(NVK * NT * 8 == CP * DK && NVV * NT * 8 == CP * DV, "staging split");
  static_assert(CT == NW || CT == NW / 2, "value tiles: one per wave, or one per block shared by both halves");
  static_assert(ELEMS * 2 == walk8_lds_elems(DK, DV, OUT) * 2, "LDS accounting");
};

// LDS of one walker workgroup, carved from one byte array: the bf16 rows, u0 (double-buffered),
// the decay table and the two halves' parts of the chunk's den.
template <int DK, int DV, bool OUT>
struct W8Lds {
  using Cfg = W8Cfg<DK, DV, OUT>;
  static constexpr int U0_OFF = Cfg::ELEMS * 2;
  static constexpr int PW_OFF = U0_OFF + 2 * DK * 4;
  static constexpr int DENS_OFF = PW_OFF + (2 * Cfg::CP + 4) * 4;
  static constexpr int BYTES = DENS_OFF + 2 * Cfg::CP * 4;
  static_assert(U0_OFF % 16 == 0 && DENS_OFF % 16 == 0, "16-byte rows");
  static_assert(BYTES == walk8_lds_bytes(DK, DV, OUT), "LDS accounting");
  static_assert(BYTES <= 160 * 1024, "one workgroup's LDS");
};

// One workgroup's walk of segment `seg` of head `bh`.  With LEAD (output mode, segment 0 of
// a plan with more than one segment) the state after the segment is written, in fp32, as
// the prefix block of segment 1, so that no summary of segment 0 is needed.
template <int DK, int DV, bool OUT, bool DEC, bool DEN, bool LEAD>
__device__ __forceinline__ void walk8_body(const WalkArgs &a, const int bh, const int seg, unsigned char *lds) {
  using Cfg = W8Cfg<DK, DV, OUT>;
  using L = W8Lds<DK, DV, OUT>;
  constexpr int CP = Cfg::CP, NB = Cfg::NB, NT = Cfg::NT, RT = Cfg::RT, KD = Cfg::KD, KC = Cfg::KC;
  constexpr int SCT = Cfg::SCT, SRT = Cfg::SRT, UCT = Cfg::UCT, NBO = Cfg::NBO;
  constexpr bool VSPLIT = Cfg::VSPLIT;
  constexpr int LDK = Cfg::LDK, LDQ = Cfg::LDQ, LDT = Cfg::LDT, LDS0 = Cfg::LDS0, LDZ = Cfg::LDZ;
  constexpr int LDV = Cfg::LDV, LDW = Cfg::LDW, NVK = Cfg::NVK, NVV = Cfg::NVV;

  bf16 *const smem = (bf16 *)lds;
  float *const pw = (float *)(lds + L::PW_OFF);      // decay^x, x = 0 .. 2 CP
  float(*const dens)[CP] = (float(*)[CP])(lds + L::DENS_OFF);  // den of the chunk's rows, per half
  float(*const u0s)[DK] = (float(*)[DK])(lds + L::U0_OFF);     // u0, double-buffered
  bf16 *const Qs = smem + Cfg::Q_OFF;
  bf16 *const Ks = smem + Cfg::K_OFF;
  bf16 *const Vs = smem + Cfg::V_OFF;
  bf16 *const Zts = smem + Cfg::ZT_OFF;
  bf16 *const Sb = smem + Cfg::SB_OFF;
  bf16 *const Zs = smem + Cfg::Z_OFF;
  bf16 *const Ws = smem + Cfg::W_OFF;
  bf16 *const Os = smem + Cfg::O_OFF;
  constexpr bool OST = Cfg::OST;
  constexpr int LDO = Cfg::LDO, NPO = Cfg::NPO;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // half and token block; at d <= 64 the second wave of SIMD w % 4 takes block 3 - (w % 4), so
  // that every SIMD holds one block near the chunk's start (few unmasked key blocks) and one near
  // its end, and the products over key blocks that the causal mask zeroes whole are skipped
  constexpr bool CSKIP = DK <= 64;
  const int hh = w >> 2, tb = (CSKIP && hh) ? 3 - (w & 3) : (w & 3);
  const int srow0 = hh * SRT;         // first d-row tile of the wave's S and Z^T tiles
  const int scol0 = tb * SCT;         // first column tile of the wave's S tiles
  const int urow = w % RT;            // u (and m) row tile; at d = 64 the second half repeats the first
  const bool u_owner = w < RT;        // writes u, m
  const bool v_owner = VSPLIT || hh == 0;  // writes its U, C tiles (at dv = 64 each half holds every tile once, as tile tb)
  const int rblk0 = VSPLIT ? 0 : 2 * hh;   // first output token block
  // value column tile j of the wave (of U, C, V and the outputs)
  auto vtile = [&](int j) __attribute__((always_inline)) -> int { return VSPLIT ? w * UCT + j : tb; };

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
  auto store_chunk = [&](int qbuf) __attribute__((always_inline)) {
    bf16 *const Qd = Qs + qbuf * CP * LDQ;
#pragma unroll
    for (int i = 0; i < NVK; ++i) {
      const int vi = tid + i * NT, t = vi / (DK / 8), e0 = 8 * (vi % (DK / 8));
      *(u32x4 *)(Qd + t * LDQ + e0) = rgq[i];
      *(u32x4 *)(Ks + t * LDK + e0) = rgk[i];
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int vi = tid + i * NT, t = vi / (DV / 8), e0 = 8 * (vi % (DV / 8));
      *(u32x4 *)(Vs + t * LDV + e0) = rgv[i];
    }
  };

  // ---------------- state ----------------
  f32x4 Sacc[SRT][SCT], Uacc[RT][UCT], uacc;
  f32x4 Cacc[OUT ? 1 : RT][OUT ? 1 : UCT], macc;
#pragma unroll
  for (int i = 0; i < SRT; ++i)
#pragma unroll
    for (int j = 0; j < SCT; ++j) Sacc[i][j] = zero4();
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < UCT; ++j) {
      Uacc[i][j] = zero4();
      if constexpr (!OUT) Cacc[i][j] = zero4();
    }
  uacc = zero4();
  macc = zero4();
  if (OUT && seg > 0) {
    // with a prologue fold (below) every segment starts from segment 1's prefix
    const int pseg = (!LEAD && DK == 64 && a.pfold) ? 1 : seg;
    const float *pb = a.prefix + ((long)bh * a.nseg + pseg) * prefix_block_floats(DK, DV);
    const float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[i][j][r] = pS[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < UCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Uacc[i][j][r] = pU[(16 * i + 4 * g + r) * DV + 16 * vtile(j) + n];
    if constexpr (DEN) {
#pragma unroll
      for (int r = 0; r < 4; ++r) uacc[r] = n == 0 ? pu[16 * urow + 4 * g + r] : 0.f;
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
  auto write_u0 = [&](int buf) __attribute__((always_inline)) {
    if constexpr (DEN) {
      if (u_owner && n == 0) *(f32x4 *)(&u0s[buf][16 * urow + 4 * g]) = uacc;
    }
  };

  // ---------------- prologue: the first chunk's loads, then the prologue fold ----------------
  load_chunk(0);

  // A three-segment lead plan has no scan launch: the workgroups of segment 2 fold segment 1's
  // summary onto segment 1's prefix with the scan's combine
  //   S <- G S + S_1,   U <- G^2 U + U_1 + G S C_1,   u <- G^2 u + u_1 + G S m_1
  // (G = decay^(tokens per segment); the cross products on bf16 MFMA from a bf16 copy of S, as
  // in the scan) while the first chunk's rows are in flight.  It runs before the loop-invariant
  // factors are formed, so its operands never share the register file with them.
  if constexpr (OUT && !LEAD && DK == 64) {
    if (a.pfold && seg == 2) {
      const float G1 = a.gamma_seg, G2 = G1 * G1;
      const float *sS = a.sums + (long)bh * walk_nsum(a) * sum_block_floats(DK, DV) + sum_block_floats(DK, DV);
      const float *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
      // C_1 in the contiguous k-order of the S rows (lane (g, n): rows 32 s + 8 g + e, column n of the tile)
      bf16x8 cb[KD][UCT], mb[KD];
#pragma unroll
      for (int s2 = 0; s2 < KD; ++s2)
#pragma unroll
        for (int j = 0; j < UCT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) cb[s2][j][e] = (bf16)sC[(32 * s2 + 8 * g + e) * DV + 16 * vtile(j) + n];
      f32x4 fu[RT][UCT], fuu = zero4();
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < UCT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) fu[i][j][q] = sU[(16 * i + 4 * g + q) * DV + 16 * vtile(j) + n];
      if constexpr (DEN) {
#pragma unroll
        for (int s2 = 0; s2 < KD; ++s2)
#pragma unroll
          for (int e = 0; e < 8; ++e) mb[s2][e] = (bf16)(n == 0 ? sm[32 * s2 + 8 * g + e] : 0.f);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float x = su[16 * urow + 4 * g + q];
          fuu[q] = n == 0 ? x : 0.f;  // u lives in column 0 of its tile
        }
      }
      write_S0();
      __syncthreads();  // the bf16 rows of S
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        bf16x8 sa[KD];
#pragma unroll
        for (int s2 = 0; s2 < KD; ++s2) sa[s2] = w8_rows_sw(Sb, LDS0, 16 * i, 32 * s2, lane);
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 mm = zero4();
#pragma unroll
          for (int s2 = 0; s2 < KD; ++s2) mm = mma(sa[s2], cb[s2][j], mm);
          Uacc[i][j] = G2 * Uacc[i][j] + fu[i][j] + G1 * mm;
        }
      }
      if constexpr (DEN) {
        f32x4 mu = zero4();
#pragma unroll
        for (int s2 = 0; s2 < KD; ++s2) mu = mma(w8_rows_sw(Sb, LDS0, 16 * urow, 32 * s2, lane), mb[s2], mu);
        uacc = G2 * uacc + fuu + G1 * mu;
      }
      __syncthreads();  // every read of the bf16 rows of S done
#pragma unroll
      for (int i = 0; i < SRT; ++i)
#pragma unroll
        for (int j = 0; j < SCT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            Sacc[i][j][q] = G1 * Sacc[i][j][q] + sS[(16 * (srow0 + i) + 4 * g + q) * DK + 16 * (scol0 + j) + n];
    }
  }

  // ---------------- loop-invariant factors ----------------
  __syncthreads();  // pw
  const int tau_w = 16 * tb + n;  // this lane's row in the wave's token block
  // A^T tile I of the wave's block: element r is (i = 16 I + 4 g + r, tau = tau_w), weight
  // [i <= tau] g^{tau - i}; the wave's W^T tiles J = 2h + jj take the square of tile J's.
  // All exponents are >= 0.
  float fa[NB][4], fw[2][4];
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * (tb - I) + n - 4 * g - r;  // tau - i
      fa[I][r] = e >= 0 ? (DEC ? pw[e] : 1.f) : 0.f;
    }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 16 * (tb - 2 * hh - jj) + n - 4 * g - r;  // tau - j
      const float x = e >= 0 ? (DEC ? pw[e] : 1.f) : 0.f;
      fw[jj][r] = x * x;
    }
  // token weights g^{63-t} of a k-step fragment (S, C and m updates): element e of k-step s
  // holds token t = 32 s + kidx(g, e)
  float kw[KC][8];
#pragma unroll
  for (int s = 0; s < KC; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) kw[s][e] = DEC ? pw[CP - 1 - (32 * s + kidx<bf16>(g, e))] : 1.f;
  const float zf = DEC ? pw[tau_w + 1] : 1.f;              // g^{tau+1}
  const float ztf = DEC ? pw[2 * (CP - 1 - tau_w)] : 1.f;  // g^{2(63-tau)}
  const float g64 = DEC ? pw[CP] : 1.f, g128 = DEC ? pw[2 * CP] : 1.f;
  // ones column (u, m): B fragment with 1 (or the token weight) in column 0
  bf16x8 ones, onesw[KC];
  {
    const bf16 o = (bf16)(n == 0 ? 1.f : 0.f);
    ones = bf16x8{o, o, o, o, o, o, o, o};
#pragma unroll
    for (int s = 0; s < KC; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) onesw[s][e] = (bf16)(n == 0 ? kw[s][e] : 0.f);
  }

  // The outputs of a chunk wait in registers and are stored at the top of the next chunk, after
  // that chunk's loads: loads and stores retire through one in-order counter, so the wait for the
  // next chunk's rows (before they go to LDS) then does not also wait for these stores.  An
  // offset past the buffer drops a store (the first chunk's, and padded columns).
  u32x2 pend[OUT ? NBO : 1][OUT ? UCT : 1];
  int poff[OUT ? NBO : 1][OUT ? UCT : 1];
#pragma unroll
  for (int rr = 0; rr < (OUT ? NBO : 1); ++rr)
#pragma unroll
    for (int j = 0; j < (OUT ? UCT : 1); ++j) {
      pend[rr][j] = u32x2{0u, 0u};
      poff[rr][j] = 0x7fffffff;
    }
  auto store_pending = [&]() __attribute__((always_inline)) {
    if constexpr (OUT && !OST) {
#pragma unroll
      for (int rr = 0; rr < NBO; ++rr)
#pragma unroll
        for (int j = 0; j < UCT; ++j) __builtin_amdgcn_raw_buffer_store_b64(pend[rr][j], ro, poff[rr][j], 0, 0);
    }
  };

  // Staged outputs (OST): the rows phase 3 left in LDS, from token trow on, as contiguous 16-byte
  // pieces; issued after the barrier that follows the next chunk's loads, so that the wait for
  // those loads does not wait for these stores either.  A row base of n drops every store.
  auto flush_out = [&](int trow) __attribute__((always_inline)) {
    if constexpr (OST) {
#pragma unroll
      for (int i = 0; i < NPO; ++i) {
        // rows of 16 pieces: lanes 0-7 and 16-23 (read together) take one whole row, so the
        // read covers the 64 banks once
        const int id = tid + i * NT, l = id & 31;
        const int row = DV / 8 == 16 ? 2 * (id >> 5) + ((l >> 3) & 1) : id / (DV / 8);
        const int cg = DV / 8 == 16 ? 8 * ((l & 7) | ((l >> 4) << 3)) : 8 * (id % (DV / 8));
        const u32x4 x = *(const u32x4 *)(Os + row * LDO + cg);
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, cg < dv ? ((trow + row) * dv + cg) * 2 : 0x7fffffff, 0, 0);
      }
    }
  };

  write_S0();
  write_u0(0);
  store_chunk(0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const bf16 *const Qc = Qs + (OUT ? (c & 1) : 0) * CP * LDQ;  // this chunk's Q
    // the next chunk's loads fly during phase 1 and land in LDS after B1
    // (a repeat of the last chunk at the end; it is never read)
    load_chunk(min(c + 1, nch - 1));
    // keep the loads here, ahead of the previous chunk's output stores: left to itself the
    // scheduler sinks them to just before B1 and waits on them at once, exposing the whole
    // memory latency every chunk
    __builtin_amdgcn_sched_barrier(0);
    store_pending();

    // ======== phase 1: chunk-local products of the wave's token block ========
    bf16x8 qw[KD];
#pragma unroll
    for (int s = 0; s < KD; ++s) qw[s] = w8_rows(Qc, LDQ, 16 * tb, 32 * s, lane);

    // A^T tiles (rows i, column tau of the block) -> masked, decayed -> Ad^T fragments.  Tiles
    // above the wave's block are zero (at d <= 64 skipped under a wave-uniform branch, else
    // computed and scaled by a zero factor).
    bf16x8 adf[KC];
    {
      f32x4 at[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        at[I] = zero4();
        if (!CSKIP || I <= tb) {  // key blocks after the wave's block are masked whole
#pragma unroll
          for (int s = 0; s < KD; ++s) at[I] = mma(w8_rows(Ks, LDK, 16 * I, 32 * s, lane), qw[s], at[I]);
#pragma unroll
          for (int r = 0; r < 4; ++r) at[I][r] *= fa[I][r];
        }
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
        kb[j][s] = ld_cols(Ks, LDK, 32 * s, 16 * (scol0 + j), lane);
        if (DEC) {
#pragma unroll
          for (int e = 0; e < 8; ++e) kb[j][s][e] = (bf16)((float)kb[j][s][e] * kw[s][e]);
        }
      }

    // per d-row tile ti of the wave, with the K^T fragments of that tile (A operand, k = tokens):
    //   Z^T tile (rows d, column tau): S0 Q_b^T scaled by g^{tau+1}, plus K^T Ad_b^T;
    //   S <- g^64 S + K^T diag(g^{63-t}) K on the wave's S tiles in that row tile.
#pragma unroll
    for (int i = 0; i < SRT; ++i) {
      const int ti = srow0 + i;
      bf16x8 kt[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) kt[s] = ld_cols(Ks, LDK, 32 * s, 16 * ti, lane);
      f32x4 z = zero4();
#pragma unroll
      for (int s = 0; s < KD; ++s) z = mma(w8_rows_sw(Sb, LDS0, 16 * ti, 32 * s, lane), qw[s], z);
      if (DEC) z *= zf;
#pragma unroll
      for (int s = 0; s < KC; ++s)
        if (!CSKIP || 32 * s <= 16 * tb + 15) z = mma(kt[s], adf[s], z);
      // Z[tau][16 ti + 4 g + r] and its decayed copy, as rows
      if constexpr (OUT) st4(Zs + tau_w * LDZ + 16 * ti + ((4 * g) ^ w8_swl(lane)), z);
      st4(Zts + tau_w * LDT + 16 * ti + ((4 * g) ^ w8_swl(lane)), DEC ? z * ztf : z);
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
      for (int s = 0; s < KC; ++s) vf[j][s] = ld_cols(Vs, LDV, 32 * s, 16 * vtile(j), lane);

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
            for (int e = 0; e < 8; ++e) vb[j][s][e] = (bf16)((float)vb[j][s][e] * kw[s][e]);
          }
        }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        bf16x8 qt[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s) qt[s] = ld_cols(Qc, LDQ, 32 * s, 16 * i, lane);
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 acc = DEC ? Cacc[i][j] * g64 : Cacc[i][j];
#pragma unroll
          for (int s = 0; s < KC; ++s) acc = mma(qt[s], vb[j][s], acc);
          Cacc[i][j] = acc;
        }
      }
      if constexpr (DEN) {
        f32x4 acc = DEC ? macc * g64 : macc;
#pragma unroll
        for (int s = 0; s < KC; ++s) acc = mma(ld_cols(Qc, LDQ, 32 * s, 16 * urow, lane), onesw[s], acc);
        macc = acc;
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

    __syncthreads();  // B1: Z, Z~ visible; every read of this chunk's K, V, S0 is done

    // ======== phase 2 ========
    // the previous chunk's staged outputs (none before the first chunk: row base n)
    flush_out(__builtin_amdgcn_readfirstlane(c > 0 ? tok0 + (c - 1) * CP : a.n));
    write_S0();
    // the next chunk's rows into LDS: this waits for their loads, so at d = 64, dv = 128 it comes
    // after the W tiles, whose products then overlap the wait (measured: decay workload 0.2313-0.2320
    // -> 0.2282-0.2295 ms; at dv = 64 and at d = 128 that order was 1% and 4% slower)
    constexpr bool LATE_STAGE = DK <= 64 && DV > 64;
    if constexpr (!LATE_STAGE) store_chunk(OUT ? ((c + 1) & 1) : 0);

    if constexpr (OUT) {
      // W^T tiles J = 2h, 2h+1 of the block (rows j, column tau) -> masked, decayed -> W rows
      // in LDS; the half's part of den
      float rs = 0.f;
      f32x4 wt[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = 2 * hh + jj;
        wt[jj] = zero4();
        if (!CSKIP || J <= tb) {
#pragma unroll
          for (int s = 0; s < KD; ++s)
            wt[jj] = mma(w8_rows_sw(Zs, LDZ, 16 * J, 32 * s, lane), qw[s], wt[jj]);
#pragma unroll
          for (int r = 0; r < 4; ++r) wt[jj][r] *= fw[jj][r];
        }
        if constexpr (DEN) rs += (wt[jj][0] + wt[jj][1]) + (wt[jj][2] + wt[jj][3]);
      }
      // tiles J = 2h and 2h + 1 of a W row sit side by side (w8_wpos): one 16-byte piece
      *(bf16x8 *)(Ws + tau_w * LDW + ((32 * hh + 8 * g) ^ w8_swl(lane))) =
          bf16x8{(bf16)wt[0][0], (bf16)wt[0][1], (bf16)wt[0][2], (bf16)wt[0][3],
                 (bf16)wt[1][0], (bf16)wt[1][1], (bf16)wt[1][2], (bf16)wt[1][3]};
      if constexpr (DEN) {
        // den_tau = g^{2(tau+1)} q_tau . u0 + sum_j W[tau][j]: the first half adds the carried term
        float qu = 0.f;
        const float *u0 = u0s[c & 1];
#pragma unroll
        for (int s = 0; s < KD; ++s) {  // qw holds k = 32 s + 8 g + 0..7
          const f32x4 ua = *(const f32x4 *)(u0 + 32 * s + 8 * g);
          const f32x4 ub = *(const f32x4 *)(u0 + 32 * s + 8 * g + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) qu += (float)qw[s][e] * ua[e] + (float)qw[s][4 + e] * ub[e];
        }
        qu = sum_groups(qu);
        rs = sum_groups(rs);
        const float part = (hh == 0 ? (DEC ? pw[2 * (tau_w + 1)] : 1.f) * qu : 0.f) + rs;
        if (g == 0) dens[hh][tau_w] = part;
      }
    }

    if constexpr (LATE_STAGE) store_chunk(OUT ? ((c + 1) & 1) : 0);

    // U <- g^128 U + Z~^T V (the wave's columns); u likewise with the ones column
    {
      bf16x8 zt[RT][KC];
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int s = 0; s < KC; ++s) zt[i][s] = w8_cols_sw(Zts, LDT, 32 * s, 16 * i, lane);
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
        f32x4 acc = DEC ? uacc * g128 : uacc;
#pragma unroll
        for (int s = 0; s < KC; ++s) acc = mma(w8_cols_sw(Zts, LDT, 32 * s, 16 * urow, lane), ones, acc);
        uacc = acc;
        if constexpr (OUT) write_u0((c + 1) & 1);
      }
    }

    __syncthreads();  // B2: W, den, the next chunk's Q, K, V and S0 visible

    // ======== phase 3: outputs (transposed tiles: rows = value columns, columns = tau) ========
    if constexpr (OUT) {
      const int t0 = tok0 + c * CP;
#pragma unroll
      for (int rr = 0; rr < NBO; ++rr) {
        const int r = rblk0 + rr;  // token block (wave-uniform)
        const float of = DEC ? pw[2 * (16 * r + n + 1)] : 1.f;
        const int t = t0 + 16 * r + n;
        float rden = 1.f;
        if constexpr (DEN) {
          const float den = dens[0][16 * r + n] + dens[1][16 * r + n];
          if (a.normalize) rden = 1.f / den;
          // den_t to the caller's buffer, by the waves holding value tile 0; rows past the end
          // fall outside the buffer and are dropped
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, den), rden_out,
                                                (g == 0 && vtile(0) == 0) ? t * 4 : 0x7fffffff, 0, 0);
        }
        // Q fragments of block r in the accumulator k-order of U0: two separate 8-byte reads per
        // fragment, each from its own opaque base
        bf16x8 qf[KD];
#pragma unroll
        for (int s = 0; s < KD; ++s) qf[s] = w8_rows_acc(Qc, LDQ, 16 * r, 32 * s, lane);
        bf16x8 wb[KC];
#pragma unroll
        for (int s = 0; s < KC; ++s)
          if (VSPLIT ? 32 * s <= 16 * rr + 15 : true) wb[s] = w8_rows_sw(Ws, LDW, 16 * r, 32 * s, lane);
#pragma unroll
        for (int j = 0; j < UCT; ++j) {
          f32x4 o = zero4();
#pragma unroll
          for (int s = 0; s < KD; ++s) o = mma(u0b[j][s], qf[s], o);
          if (DEC) o *= of;
#pragma unroll
          for (int s = 0; s < KC; ++s)
            if (VSPLIT ? 32 * s <= 16 * rr + 15 : true) o = mma(vf[j][s], wb[s], o);
          if (DEN) o *= rden;
          const bf16x4 ob = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
          // stored at the top of the next chunk (or after the loop); rows past the end fall
          // outside the buffer, and padded columns are sent there too
          const int col = 16 * vtile(j) + 4 * g;
          if constexpr (OST) {
            *(bf16x4 *)(Os + (16 * r + n) * LDO + col) = ob;
          } else {
            pend[rr][j] = __builtin_bit_cast(u32x2, ob);
            poff[rr][j] = col < dv ? (t * dv + col) * 2 : 0x7fffffff;
          }
        }
      }
    }
  }

  store_pending();  // the last chunk's outputs
  if constexpr (OST) {
    __syncthreads();  // the last chunk's staged rows
    flush_out(tok0 + (nch - 1) * CP);
  }

  // ---------------- segment summary: S | C | U | m | u ----------------
  if constexpr (!OUT) {
    float *sb = a.sums + ((long)bh * walk_nsum(a) + seg) * sum_block_floats(DK, DV);
    float *sS = sb, *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n] = Sacc[i][j][r];
    if (v_owner) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < UCT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sC[(16 * i + 4 * g + r) * DV + 16 * vtile(j) + n] = Cacc[i][j][r];
            sU[(16 * i + 4 * g + r) * DV + 16 * vtile(j) + n] = Uacc[i][j][r];
          }
    }
    if (u_owner && n == 0) {
      *(f32x4 *)(sm + 16 * urow + 4 * g) = DEN ? macc : zero4();
      *(f32x4 *)(su + 16 * urow + 4 * g) = DEN ? uacc : zero4();
    }
  }

  // ---------------- lead segment: its final state is the prefix S0 | U0 | u0 of segment 1 ----------------
  // (the layout the prefix is read in above; u0 is zero when den is not carried)
  if constexpr (OUT && LEAD) {
    float *pb = a.prefix_out + ((long)bh * a.nseg + seg + 1) * prefix_block_floats(DK, DV);
    float *pS = pb, *pU = pb + DK * DK, *pu = pU + DK * DV;
#pragma unroll
    for (int i = 0; i < SRT; ++i)
#pragma unroll
      for (int j = 0; j < SCT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) pS[(16 * (srow0 + i) + 4 * g + r) * DK + 16 * (scol0 + j) + n] = Sacc[i][j][r];
    if (v_owner) {
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < UCT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) pU[(16 * i + 4 * g + r) * DV + 16 * vtile(j) + n] = Uacc[i][j][r];
    }
    if (u_owner && n == 0) *(f32x4 *)(pu + 16 * urow + 4 * g) = DEN ? uacc : zero4();
  }
}

// Walks segments seg_lo .. (nseg or nsum) - 1 of every head, one workgroup each.  One
// workgroup of eight waves per CU: two waves per SIMD, 256 registers each.
template <int DK, int DV, bool OUT, bool DEC, bool DEN>
__global__ void __launch_bounds__(512, 2) walk8_kernel(WalkArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[W8Lds<DK, DV, OUT>::BYTES];
  const int nr = (OUT ? a.nseg : walk_nsum(a)) - a.seg_lo;  // segments of a head in this launch
  walk8_body<DK, DV, OUT, DEC, DEN, false>(a, blockIdx.x / nr, a.seg_lo + blockIdx.x % nr, lds);
}

// The lead launch: workgroups 0 .. nbh-1 walk segment 0 of their head in output mode and
// leave the prefix of segment 1; the rest summarise segments 1 .. nsum-1 of every head.
// Both roles share one LDS allocation (the larger, output mode's).
template <int DK, int DV, bool DEC, bool DEN>
__global__ void __launch_bounds__(512, 2) walk8_lead_kernel(WalkArgs a) {
  constexpr int BO = W8Lds<DK, DV, true>::BYTES, BS = W8Lds<DK, DV, false>::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char lds[BO > BS ? BO : BS];
  const int b = blockIdx.x;
  if (b < a.nbh) {
    walk8_body<DK, DV, true, DEC, DEN, true>(a, b, 0, lds);
  } else {
    const int i = b - a.nbh, nr = walk_nsum(a) - 1;
    walk8_body<DK, DV, false, DEC, DEN, false>(a, i / nr, 1 + i % nr, lds);
  }
}

template <int DK, int DV>
hipError_t launch_walk8_t(bool out, bool dec, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
#define HLA2_W8(O, D, N)                                                                     \
  if (out == O && dec == D && den == N) {                                                    \
    hipLaunchKernelGGL((walk8_kernel<DK, DV, O, D, N>), grid, dim3(512), 0, s, a);          \
    return hipGetLastError();                                                                \
  }
  HLA2_W8(true, true, true)
  HLA2_W8(true, true, false)
  HLA2_W8(true, false, true)
  HLA2_W8(true, false, false)
  HLA2_W8(false, true, true)
  HLA2_W8(false, true, false)
  HLA2_W8(false, false, true)
  HLA2_W8(false, false, false)
#undef HLA2_W8
  return hipErrorInvalidValue;
}

template <int DK, int DV>
hipError_t launch_walk8_lead_t(bool dec, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
#define HLA2_W8L(D, N)                                                                       \
  if (dec == D && den == N) {                                                                \
    hipLaunchKernelGGL((walk8_lead_kernel<DK, DV, D, N>), grid, dim3(512), 0, s, a);        \
    return hipGetLastError();                                                                \
  }
  HLA2_W8L(true, true)
  HLA2_W8L(true, false)
  HLA2_W8L(false, true)
  HLA2_W8L(false, false)
#undef HLA2_W8L
  return hipErrorInvalidValue;
}

}  // namespace hla2
