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
// tiles and heads run in parallel.  The S0 C_r product runs on fp32 MFMA, and
// the loads of step r+1 are issued before step r is computed.
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

template <int DK, int DV>
__global__ void __launch_bounds__(64) scan_kernel(ScanArgs a) {
  // MFMA k-order: for step (jj, e) lane group g holds k = 16 jj + 4 g + e, so a
  // lane's share of an S0 row is DK/16 contiguous float4s.
  constexpr int NJ = DK / 16;
  constexpr int CU = DV / 16;  // column tile index of the u column
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
    const float *sb = sums + ((long)bh * (a.nseg - 1) + r) * SB;
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

  f32x4 sr[NJ], cr[NJ], loc;
  if (a.nseg > 1) load(0, sr, cr, loc);
  for (int r = 0; r < a.nseg; ++r) {
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
    if (r == a.nseg - 1) break;
    f32x4 srn[NJ], crn[NJ], locn;
    if (r + 1 < a.nseg - 1) load(r + 1, srn, crn, locn);  // prefetch the next step
    f32x4 mm = zero4();
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) mm = mfma_f32_guarded(s0[jj][e], cr[jj][e], mm);
    acc = G2 * acc + loc + G1 * mm;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) s0[jj] = G1 * s0[jj] + sr[jj];
    if (r + 1 < a.nseg - 1) {
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        sr[jj] = srn[jj];
        cr[jj] = crn[jj];
      }
      loc = locn;
    }
  }
}

template <int DK, int DV>
static hipError_t launch_scan_t(int BH, const ScanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((scan_kernel<DK, DV>), dim3(BH, DK / 16, DV / 16 + 1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(int DK, int DV, int BH, const ScanArgs &a, hipStream_t s) {
  if (DK == 16 && DV == 16) return launch_scan_t<16, 16>(BH, a, s);
  if (DK == 64 && DV == 64) return launch_scan_t<64, 64>(BH, a, s);
  if (DK == 64 && DV == 128) return launch_scan_t<64, 128>(BH, a, s);
  if (DK == 128 && DV == 64) return launch_scan_t<128, 64>(BH, a, s);
  if (DK == 128 && DV == 128) return launch_scan_t<128, 128>(BH, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_walk(int dtype, int DK, int DV, int CP, bool output_mode, dim3 grid,
                       const WalkArgs &a, hipStream_t s) {
  if (dtype == 0) return launch_walk_f32(DK, DV, CP, output_mode, grid, a, s);
  if (CP != 64) return hipErrorInvalidValue;
  const bool dec = a.decay_on != 0, den = a.need_den != 0;
  if (DK == 64) return launch_walk3_dk64(DV, output_mode, dec, den, grid, a, s);
  if (DK == 128) return launch_walk3_dk128(DV, output_mode, dec, den, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
