// hla2_scan.hip -- exclusive scan over segment summaries, and the walker
// dispatcher.
//
// Segments A then B concatenate by the semidirect-product rule of the
// technical summary of arXiv 2510.27258 (gist.science, §4 "Associatieve
// operatoren"), written here for the corrected state U = S C - G:
//   S_AB = g_B S_A + S_B
//   C_AB = g_B C_A + C_B
//   U_AB = g_B^2 U_A + U_B + g_B S_A C_B      (u likewise with m_B)
// where g_B = decay^(length of B).  (In the G form the cross term is
// g_B S_B C_A; the two agree because U = S C - G.)  The exclusive prefix of
// segment r is P_r = seg_0 ... seg_{r-1}; P_0 is the zero state.  Only S and U
// (and u) of the prefixes are needed downstream, so the scan runs
//   S0_{r+1} = g S0_r + S_r,   U0_{r+1} = g^2 U0_r + U_r + g S0_r C_r,
// every full segment having the same length.  One wave owns a 16x16 tile of U0
// (or the 16-row slice of u0) and the matching 16-row slice of S0, and walks r;
// tiles and heads run in parallel.  The S0 C_r product runs on fp32 MFMA.  Steps
// have no loads that depend on earlier steps, so the loads of PF consecutive steps
// are issued together and the walk pays one memory latency per PF steps.
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

// fp32 path (fp32 inputs, d <= 64): one wave per (head, 16-row tile, column tile),
// fp32 MFMA for the cross term.
template <int DK, int DV>
__global__ void __launch_bounds__(64) scan_kernel(ScanArgs a) {
  // MFMA k-order: for step (jj, e) lane group g holds k = 16 jj + 4 g + e, so a
  // lane's share of an S0 row is DK/16 contiguous float4s.
  constexpr int NJ = DK / 16;
  constexpr int CU = DV / 16;         // column tile index of the u column
  constexpr int PF = DK == 64 ? 4 : 2;  // steps whose loads are in flight together
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, rt = blockIdx.y, ct = blockIdx.z;
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  const float G1 = a.gamma_seg, G2 = a.gamma_seg * a.gamma_seg;
  const float *__restrict__ sums = a.sums;
  float *__restrict__ prefix = a.prefix;

  f32x4 s0[NJ];  // S0[16 rt + n][16 jj + 4 g + e]
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) s0[jj] = zero4();
  f32x4 acc = zero4();  // U0[16 rt + 4 g + q][16 ct + n]   (or u0[16 rt + 4 g + q] in column n = 0)

  // the loads of one step: rows of S_r, a column tile of C_r (or m_r), a tile of U_r (or u_r)
  auto load = [&](int r, f32x4 (&sr)[NJ], f32x4 (&cr)[NJ], f32x4 &loc) __attribute__((always_inline)) {
    const float *sb = sums + ((long)bh * a.nsum + r) * SB;
    const float *sS = sb, *sC = sS + DK * DK, *sU = sC + DK * DV, *sm = sU + DK * DV, *su = sm + DK;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      sr[jj] = *(const f32x4 *)(sS + (16 * rt + n) * DK + 16 * jj + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 16 * jj + 4 * g + e;
        cr[jj][e] = (ct < CU) ? sC[k * DV + 16 * ct + n] : (n == 0 ? sm[k] : 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      loc[q] = (ct < CU) ? sU[(16 * rt + 4 * g + q) * DV + 16 * ct + n] : (n == 0 ? su[16 * rt + 4 * g + q] : 0.f);
  };
  // write the exclusive prefix of segment r (the state before it)
  auto store = [&](int r) __attribute__((always_inline)) {
    float *pb = prefix + ((long)bh * a.nseg + r) * PB;
    if (ct == 0) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) *(f32x4 *)(pb + (16 * rt + n) * DK + 16 * jj + 4 * g) = s0[jj];
    }
    if (ct < CU) {
#pragma unroll
      for (int q = 0; q < 4; ++q) pb[DK * DK + (16 * rt + 4 * g + q) * DV + 16 * ct + n] = acc[q];
    } else if (n == 0) {
      *(f32x4 *)(pb + DK * DK + DK * DV + 16 * rt + 4 * g) = acc;
    }
  };

  const int steps = a.nseg - 1;  // segment summaries to fold in
  for (int r0 = 0; r0 < steps; r0 += PF) {
    f32x4 sr[PF][NJ], cr[PF][NJ], loc[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (r0 + j < steps) load(r0 + j, sr[j], cr[j], loc[j]);
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      if (r0 + j < steps) {
        store(r0 + j);
        f32x4 mm = zero4();
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) mm = mfma_f32_guarded(s0[jj][e], cr[j][jj][e], mm);
        acc = G2 * acc + loc[j] + G1 * mm;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) s0[jj] = G1 * s0[jj] + sr[j][jj];
      }
    }
  }
  store(steps);
}

// Column groups (workgroups per head) of the bf16 scan: each keeps all of S0 and owns DV/4 value
// columns.  The walk is a chain of latency-bound steps; against two groups, four put twice the
// loads in flight with a smaller share each (measured: long 64k workload's scan 74.5 -> 64.7 us,
// normalised 2k 12.4 -> 11.7 us).
__host__ __device__ constexpr int scan_groups(int) { return 4; }

// bf16 path: scan_groups(DK) workgroups per head, each owning a slice of the value columns (the
// last also the u column) for all rows, with one wave per 16-row tile.  The cross term S0 C_r
// runs on bf16 MFMA, like every other state product of the bf16 walkers: each step the
// group's columns of C_r (and m_r) are converted to bf16 into LDS once and read by every
// wave, while the next step's C_r is already being fetched.
template <int DK, int DV>
__global__ void __launch_bounds__(64 * (DK / 16)) scan_bf16_kernel(ScanArgs a) {
  constexpr int NWV = DK / 16;        // waves = row tiles
  constexpr int NT = 64 * NWV;
  constexpr int NJ = DK / 16;         // f32x4 per lane of an S0 row
  constexpr int NG = scan_groups(DK);
  constexpr int HC = DV / NG;         // value columns per workgroup
  constexpr int CT = HC / 16;         // value column tiles per workgroup
  constexpr int LDC = HC + 16;        // bf16 C_r rows: HC values, then m_r (last group), zeros
  constexpr int NC4 = DK * HC / 4 / NT;  // f32x4 of C_r per thread
  static_assert(NC4 * 4 * NT == DK * HC, "C staging split");
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, grp = blockIdx.y, c0 = grp * HC;  // first value column
  const bool has_u = grp == NG - 1;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float G1 = a.gamma_seg, G2 = a.gamma_seg * a.gamma_seg;
  __shared__ __attribute__((aligned(16))) bf16 Cb[2][DK * LDC];

  // columns HC .. HC+15 hold m_r (column HC, last group) and zeros; zero them once
  for (int x = tid; x < 2 * DK * 16; x += NT) {
    const int b = x / (DK * 16), r = (x / 16) % DK, c = HC + x % 16;
    Cb[b][r * LDC + c] = (bf16)0.f;
  }
  // the fill writes column HC of rows that other waves own; the first step's m_r goes into
  // that column, so every zero must land before any thread writes it
  __syncthreads();

  f32x4 s0[NJ];       // S0[16 w + n][16 jj + 4 g + e]
  f32x4 acc[CT + 1];  // U0[16 w + 4 g + q][c0 + 16 ct + n]; tile CT holds u0 in column 0
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) s0[jj] = zero4();
#pragma unroll
  for (int ct = 0; ct <= CT; ++ct) acc[ct] = zero4();

  // loads of one step: the group's C_r columns and m_r (staged into LDS at the top of the
  // step, so they are fetched one step ahead) and the wave's rows of S_r and U_r
  f32x4 cr[NC4], sr[NJ], lr[CT + 1];
  float mr = 0.f;
  auto block = [&](int r) __attribute__((always_inline)) {
    return a.sums + ((long)bh * a.nsum + r) * SB;
  };
  auto load_c = [&](int r) __attribute__((always_inline)) {
    const float *sC = block(r) + DK * DK, *sm = sC + 2 * DK * DV;
#pragma unroll
    for (int i = 0; i < NC4; ++i) {
      const int e = 4 * (tid + i * NT), row = e / HC, col = e % HC;
      cr[i] = *(const f32x4 *)(sC + row * DV + c0 + col);
    }
    if (has_u && tid < DK) mr = sm[tid];
  };
  auto load_su = [&](int r) __attribute__((always_inline)) {
    const float *sS = block(r), *sU = sS + DK * DK + DK * DV, *su = sU + DK * DV + DK;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) sr[jj] = *(const f32x4 *)(sS + (16 * w + n) * DK + 16 * jj + 4 * g);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) lr[ct][q] = sU[(16 * w + 4 * g + q) * DV + c0 + 16 * ct + n];
#pragma unroll
    for (int q = 0; q < 4; ++q) lr[CT][q] = (has_u && n == 0) ? su[16 * w + 4 * g + q] : 0.f;
  };
  // the exclusive prefix of segment r (S0 rows written by the first group only)
  auto store = [&](int r) __attribute__((always_inline)) {
    if (r < a.pmin) return;
    float *pb = a.prefix + ((long)bh * (a.pnseg > 0 ? a.pnseg : a.nseg) + r - a.pshift) * PB;
    if (grp == 0) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) *(f32x4 *)(pb + (16 * w + n) * DK + 16 * jj + 4 * g) = s0[jj];
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) pb[DK * DK + (16 * w + 4 * g + q) * DV + c0 + 16 * ct + n] = acc[ct][q];
    if (has_u && n == 0) *(f32x4 *)(pb + DK * DK + DK * DV + 16 * w + 4 * g) = acc[CT];
  };

  const int steps = a.nseg - 1;
  const int r0 = a.first;  // with a given prefix of segment 1 the fold starts from it
  if (r0 > 0) {
    const float *pb = a.prefix + ((long)bh * a.nseg + r0) * PB;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) s0[jj] = *(const f32x4 *)(pb + (16 * w + n) * DK + 16 * jj + 4 * g);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[ct][q] = pb[DK * DK + (16 * w + 4 * g + q) * DV + c0 + 16 * ct + n];
    if (has_u && n == 0) acc[CT] = *(const f32x4 *)(pb + DK * DK + DK * DV + 16 * w + 4 * g);
  }
  load_c(r0);
  for (int r = r0; r < steps; ++r) {
    load_su(r);
    bf16 *cb = Cb[r & 1];
#pragma unroll
    for (int i = 0; i < NC4; ++i) {
      const int e = 4 * (tid + i * NT), row = e / HC, col = e % HC;
      st4(cb + row * LDC + col, cr[i]);
    }
    if (has_u && tid < DK) cb[tid * LDC + HC] = (bf16)mr;
    __syncthreads();  // C_r visible; the other buffer is free again
    if (r + 1 < steps) load_c(r + 1);

    if (r > r0 || r0 == 0) store(r);  // a given prefix is already in place
    bf16x8 af[DK / 32];
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) af[s] = frag_from_acc(s0[2 * s], s0[2 * s + 1]);
#pragma unroll
    for (int ct = 0; ct <= CT; ++ct) {
      f32x4 mm = zero4();
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) mm = mma(af[s], ld_cols(cb, LDC, 32 * s, 16 * ct, lane), mm);
      acc[ct] = G2 * acc[ct] + lr[ct] + G1 * mm;
    }
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) s0[jj] = G1 * s0[jj] + sr[jj];
  }
  store(steps);
}

// ---------------------------------------------------------------------------------------------
// Parallel form of the same exclusive scan (bf16 path, forward plans).  With every folded segment
// of the same length (factor G), the prefix recurrences separate:
//   S0_{r+1} = G S0_r + S_r                       a decayed prefix sum of the S summaries;
//   U0_{r+1} = G^2 U0_r + T_r,  T_r = U_r + G S0_r C_r   (u likewise with m_r)
// so the cross products S0_r C_r, which carry all the arithmetic, are independent once every
// S0_r is known.  Three launches of constant depth replace the chain of steps:
//   scan_s_kernel     the S0 prefix sums (elementwise over r),
//   scan_t_kernel     every T_r, t_r at once (bf16 MFMA, as the fold), written over U_r, u_r in
//                     the summary blocks (which nothing reads afterwards),
//   scan_u_kernel     the U0, u0 prefix sums (elementwise over r).
// The steps fold summaries r0 .. steps-1 (r0 = first), and write prefixes r0+1 .. steps (and the
// zero prefix 0 when r0 = 0).
constexpr int SCAN_ELEM_THREADS = 256;

// S0 prefix: thread x owns one f32x4 of S (d x d) of one head.
template <int DK, int DV>
__global__ void __launch_bounds__(SCAN_ELEM_THREADS) scan_s_kernel(ScanArgs a) {
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, e = 4 * (blockIdx.y * SCAN_ELEM_THREADS + threadIdx.x);
  if (e >= DK * DK) return;
  const float G = a.gamma_seg;
  const int r0 = a.first, steps = a.nseg - 1;
  float *pref = a.prefix + (long)bh * a.nseg * PB;
  const float *sums = a.sums + (long)bh * a.nsum * SB;
  f32x4 s0 = r0 > 0 ? *(const f32x4 *)(pref + r0 * PB + e) : zero4();
  if (r0 == 0) *(f32x4 *)(pref + e) = s0;
  for (int r = r0; r < steps; r += 8) {
    f32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = r + j < steps ? *(const f32x4 *)(sums + (r + j) * SB + e) : zero4();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r + j < steps) {
        s0 = G * s0 + x[j];
        *(f32x4 *)(pref + (r + j + 1) * PB + e) = s0;
      }
    }
  }
}

// U0 and u0 prefix: thread x owns one f32x4 of U (d x dv) or of u (d) of one head.
template <int DK, int DV>
__global__ void __launch_bounds__(SCAN_ELEM_THREADS) scan_u_kernel(ScanArgs a) {
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, e = 4 * (blockIdx.y * SCAN_ELEM_THREADS + threadIdx.x);
  if (e >= DK * DV + DK) return;
  const float G2 = a.gamma_seg * a.gamma_seg;
  const int r0 = a.first, steps = a.nseg - 1;
  // U0 | u0 are contiguous in a prefix block; in a summary block T (over U) is followed by m, then t
  const int po = DK * DK + e, so = e < DK * DV ? DK * DK + DK * DV + e : DK * DK + 2 * DK * DV + DK + (e - DK * DV);
  float *pref = a.prefix + (long)bh * a.nseg * PB;
  const float *sums = a.sums + (long)bh * a.nsum * SB;
  f32x4 u0 = r0 > 0 ? *(const f32x4 *)(pref + r0 * PB + po) : zero4();
  if (r0 == 0) *(f32x4 *)(pref + po) = u0;
  for (int r = r0; r < steps; r += 8) {
    f32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = r + j < steps ? *(const f32x4 *)(sums + (r + j) * SB + so) : zero4();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r + j < steps) {
        u0 = G2 * u0 + x[j];
        *(f32x4 *)(pref + (r + j + 1) * PB + po) = u0;
      }
    }
  }
}

// T_r = U_r + G S0_r C_r (and t_r = u_r + G S0_r m_r) for one folded summary r (blockIdx.y, from
// r0) and one group of value columns (blockIdx.z; the last group also t_r); one wave per 16-row
// tile of S0, C_r's columns staged in LDS as bf16.
template <int DK, int DV>
__global__ void __launch_bounds__(64 * (DK / 16)) scan_t_kernel(ScanArgs a) {
  constexpr int NT = 64 * (DK / 16);
  constexpr int NJ = DK / 16;
  constexpr int NG = scan_groups(DK);
  constexpr int HC = DV / NG, CT = HC / 16, LDC = HC + 16;
  constexpr int NC4 = DK * HC / 4 / NT;
  static_assert(NC4 * 4 * NT == DK * HC, "C staging split");
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, r = a.first + blockIdx.y, grp = blockIdx.z, c0 = grp * HC;
  const bool has_u = grp == NG - 1;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float G = a.gamma_seg;
  __shared__ __attribute__((aligned(16))) bf16 Cb[DK * LDC];
  float *sb = a.sums + ((long)bh * a.nsum + r) * SB;
  const float *sC = sb + DK * DK, *sm = sC + 2 * DK * DV;
  float *sU = sb + DK * DK + DK * DV, *su = sU + DK * DV + DK;
  const float *pS = a.prefix + ((long)bh * a.nseg + r) * PB;
  // C_r's columns (and m_r in column HC of the last group; zeros elsewhere) into LDS
#pragma unroll
  for (int i = 0; i < NC4; ++i) {
    const int e = 4 * (tid + i * NT), row = e / HC, col = e % HC;
    st4(Cb + row * LDC + col, *(const f32x4 *)(sC + row * DV + c0 + col));
  }
  for (int x = tid; x < DK * 16; x += NT) {
    const int row = x / 16, col = x % 16;
    Cb[row * LDC + HC + col] = (bf16)((has_u && col == 0) ? sm[row] : 0.f);
  }
  // the wave's rows of S0_r as bf16 A fragments, and its tiles of U_r (u_r)
  bf16x8 af[DK / 32];
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    const f32x4 lo = *(const f32x4 *)(pS + (16 * w + n) * DK + 32 * s + 4 * g);
    const f32x4 hi = *(const f32x4 *)(pS + (16 * w + n) * DK + 32 * s + 16 + 4 * g);
    af[s] = frag_from_acc(lo, hi);
  }
  f32x4 ur[CT + 1];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) ur[ct][q] = sU[(16 * w + 4 * g + q) * DV + c0 + 16 * ct + n];
#pragma unroll
  for (int q = 0; q < 4; ++q) ur[CT][q] = (has_u && n == 0) ? su[16 * w + 4 * g + q] : 0.f;
  __syncthreads();  // C_r staged
#pragma unroll
  for (int ct = 0; ct <= CT; ++ct) {
    f32x4 mm = zero4();
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) mm = mma(af[s], ld_cols(Cb, LDC, 32 * s, 16 * ct, lane), mm);
    ur[ct] = ur[ct] + G * mm;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) sU[(16 * w + 4 * g + q) * DV + c0 + 16 * ct + n] = ur[ct][q];
  if (has_u && n == 0) *(f32x4 *)(su + 16 * w + 4 * g) = ur[CT];
}

// The parallel form takes the forward plans with at least this many folded summaries; shorter
// scans (and the backward's split prefix) keep the fold.  Measured: 15 folds at d = dv = 128, 65 ->
// 30 us; 6 folds at d = dv = 64, the fold is faster than the three launches.
constexpr int SCAN_PAR_MIN_STEPS = 8;

template <int DK, int DV>
static hipError_t launch_scan_t(int BH, bool bf, const ScanArgs &a, hipStream_t s) {
  if (a.first != 0 && !(bf && DK >= 64)) return hipErrorInvalidValue;  // only the bf16 fold takes a given prefix
  if (a.first < 0 || a.first > 1 || (a.first == 1 && a.nseg < 3)) return hipErrorInvalidValue;
  if ((a.pnseg != 0 || a.pmin != 0 || a.pshift != 0) && !(bf && DK >= 64)) return hipErrorInvalidValue;
  if (a.pshift < 0 || a.pshift > a.pmin) return hipErrorInvalidValue;
  if constexpr (DK >= 64) {
    if (bf) {
      const int folds = a.nseg - 1 - a.first;
      if (folds >= SCAN_PAR_MIN_STEPS && a.pnseg == 0 && a.pmin == 0 && a.pshift == 0) {
        const int nbs = (DK * DK / 4 + SCAN_ELEM_THREADS - 1) / SCAN_ELEM_THREADS;
        const int nbu = ((DK * DV + DK) / 4 + SCAN_ELEM_THREADS - 1) / SCAN_ELEM_THREADS;
        hipLaunchKernelGGL((scan_s_kernel<DK, DV>), dim3(BH, nbs), dim3(SCAN_ELEM_THREADS), 0, s, a);
        hipLaunchKernelGGL((scan_t_kernel<DK, DV>), dim3(BH, folds, scan_groups(DK)), dim3(64 * (DK / 16)), 0, s, a);
        hipLaunchKernelGGL((scan_u_kernel<DK, DV>), dim3(BH, nbu), dim3(SCAN_ELEM_THREADS), 0, s, a);
        return hipGetLastError();
      }
      hipLaunchKernelGGL((scan_bf16_kernel<DK, DV>), dim3(BH, scan_groups(DK)), dim3(64 * (DK / 16)), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((scan_kernel<DK, DV>), dim3(BH, DK / 16, DV / 16 + 1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(int dtype, int DK, int DV, int BH, const ScanArgs &a, hipStream_t s) {
  const bool bf = dtype != 0;
  if (DK == 16 && DV == 16) return launch_scan_t<16, 16>(BH, false, a, s);
  if (DK == 64 && DV == 64) return launch_scan_t<64, 64>(BH, bf, a, s);
  if (DK == 64 && DV == 128) return launch_scan_t<64, 128>(BH, bf, a, s);
  if (DK == 128 && DV == 64) return launch_scan_t<128, 64>(BH, bf, a, s);
  if (DK == 128 && DV == 128) return launch_scan_t<128, 128>(BH, bf, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_walk_lead(int DK, int DV, dim3 grid, const WalkArgs &a, hipStream_t s) {
  const bool dec = a.decay_on != 0, den = a.need_den != 0;
  if (a.nseg < 2 || a.sum_all || a.nbh < 1 || !a.prefix_out) return hipErrorInvalidValue;
  if (DK == 64) return launch_walk8_lead_dk64(DV, dec, den, grid, a, s);
  if (DK == 128) return launch_walk8_lead_dk128(DV, dec, den, grid, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_walk(int dtype, int DK, int DV, int CP, bool output_mode, dim3 grid,
                       const WalkArgs &a, hipStream_t s) {
  if (dtype == 0) return launch_walk_f32(DK, DV, CP, output_mode, grid, a, s);
  if (CP != 64) return hipErrorInvalidValue;
  const bool dec = a.decay_on != 0, den = a.need_den != 0;
  if (DK == 64) return launch_walk8_dk64(DV, output_mode, dec, den, grid, a, s);
  if (DK == 128) return launch_walk8_dk128(DV, output_mode, dec, den, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
