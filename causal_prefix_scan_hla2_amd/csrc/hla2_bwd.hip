// hla2_bwd.hip -- the backward pass: upstream-gradient preparation for the
// ratio, the reverse scan over segments, and the instantiations and launchers
// of the backward walkers (hla2_bwd.h).
#include "hla2_bwd.h"

namespace hla2 {

// Upstream gradient of [num | den] under the ratio o = num / den:
//   g'[t][c] = dout[t][c] / den[t]  (c < dv),   g'[t][DV] = -(dout[t] . out[t]) / den[t],
// zero elsewhere; rows of DVP elements.  One wave per token.
template <typename T, int DV, int DVP>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdPrepArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const T *g = (const T *)a.dout + row * a.dv, *o = (const T *)a.out + row * a.dv;
  T *gp = (T *)a.gprep + row * DVP;
  const float inv = 1.f / a.den[row];
  float dot = 0.f;
  for (int c = lane; c < a.dv; c += 64) dot += (float)g[c] * (float)o[c];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
  for (int c = lane; c < DVP; c += 64) {
    float x = 0.f;
    if (c < a.dv) x = (float)g[c] * inv;
    else if (c == DV) x = -dot * inv;
    gp[c] = (T)x;
  }
}

// Reverse (adjoint) scan over segments, per (b, h): the adjoint state at the end
// of segment r is the fold of the adjoint summaries of the later segments,
//   Ubar <- g^(2L) Ubar + Ubar_r,
//   Shat <- g^L Shat + Shat_r + g^(L+1) (Ubar C'_r^T + C'_r Ubar^T)   (old Ubar),
// taken from the last segment backwards; L = tokens per full segment and
// C'_r = [C_r | m_r] the segment's forward summary.  fp32 on VALU.
// Workgroup (bh, sp) owns rows 16 sp .. 16 sp + 15 of Shat; every workgroup of a
// head keeps the whole Ubar sequence itself (elementwise and cheap), so the
// workgroups never wait on each other.  Ubar is written by the sp = 0 group.
template <int DK, int DV, int DVP, bool NORM>
__global__ void __launch_bounds__(256) bwd_rscan_kernel(BwdArgs a, float gL) {
  constexpr int CW = DVP / 2;                     // columns of C' staged per pass
  constexpr long RB = (long)DK * DVP + DK * DK;   // adjoint block
  constexpr int NU = (DK * DVP + 255) / 256;      // Ubar elements per thread
  constexpr int NO = 16 * DK / 256 > 0 ? 16 * DK / 256 : 1;  // Shat entries per thread (one row, NO columns)
  __shared__ __attribute__((aligned(16))) float Us[DK * DVP], Cs[DK * CW];
  const int tid = threadIdx.x, bh = blockIdx.x, sp = blockIdx.y;
  // thread -> (row a in the group's 16, columns b0 .. b0 + NO - 1)
  const bool active = tid * NO < 16 * DK;
  const int a_row = 16 * sp + (active ? (tid * NO) / DK : 0), b0 = active ? (tid * NO) % DK : 0;
  const long SB = sum_block_floats(DK, DV);
  float *suf = a.suffix + (long)bh * a.nseg * RB;
  const float *rs = a.rsum + (long)bh * a.nseg * RB;
  const float gL1 = gL * exp2f(a.log2g), gL2 = gL * gL;
  float U[NU], Sh[NO];
#pragma unroll
  for (int i = 0; i < NU; ++i) U[i] = 0.f;
#pragma unroll
  for (int o = 0; o < NO; ++o) Sh[o] = 0.f;
  auto store = [&](int r) {
    float *out = suf + (long)r * RB;
    if (sp == 0) {
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int e = tid + 256 * i;
        if (e < DK * DVP) out[e] = U[i];
      }
    }
    if (active) {
#pragma unroll
      for (int o = 0; o < NO; ++o) out[DK * DVP + a_row * DK + b0 + o] = Sh[o];
    }
  };
  store(a.nseg - 1);
  for (int r = a.nseg - 1; r >= 1; --r) {
    const float *ad = rs + (long)r * RB;
    float X[NO];
#pragma unroll
    for (int o = 0; o < NO; ++o) X[o] = 0.f;
    if (r < a.nseg - 1) {  // the cross term with the old Ubar (zero before the first fold)
      const float *fs = a.fsum + ((long)bh * (a.nseg - 1) + r) * SB;
      const float *Cg = fs + DK * DK, *mg = fs + DK * DK + 2 * DK * DV;
      __syncthreads();  // the previous step's reads of Us are done
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int e = tid + 256 * i;
        if (e < DK * DVP) Us[e] = U[i];
      }
      for (int h = 0; h < 2; ++h) {
        __syncthreads();
        for (int e = tid; e < DK * CW; e += 256) {
          const int row = e / CW, c = h * CW + e % CW;
          Cs[e] = c < DV ? Cg[row * DV + c] : ((NORM && c == DV) ? mg[row] : 0.f);
        }
        __syncthreads();
        if (active) {
          for (int c = 0; c < CW; ++c) {
            const float ua = Us[a_row * DVP + h * CW + c], ca = Cs[a_row * CW + c];
#pragma unroll
            for (int o = 0; o < NO; ++o)
              X[o] += ua * Cs[(b0 + o) * CW + c] + ca * Us[(b0 + o) * DVP + h * CW + c];
          }
        }
      }
    }
    if (active) {
#pragma unroll
      for (int o = 0; o < NO; ++o) Sh[o] = gL * Sh[o] + ad[DK * DVP + a_row * DK + b0 + o] + gL1 * X[o];
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int e = tid + 256 * i;
      if (e < DK * DVP) U[i] = gL2 * U[i] + ad[e];
    }
    store(r - 1);
  }
}

// ---------------------------------------------------------------------------
// Launchers.  The backward walkers hold one workgroup per CU (their LDS), so
// each may use every register of its SIMD.
template <typename T, int DK, int DV, bool NORM>
struct BwdShape {
  static constexpr int DVP = lds_walk_dvp(sizeof(T) == 4, DV, NORM);
  static constexpr int BC = lds_bwd_chunk(sizeof(T) == 4, DK, DVP);
};

template <typename T, int DK, int DV, bool NORM>
static hipError_t launch_bwd_t(int phase, int BH, const BwdArgs &a, const BwdPrepArgs &pa, float gL, hipStream_t s) {
  using Sh = BwdShape<T, DK, DV, NORM>;
  constexpr int DVP = Sh::DVP, BC = Sh::BC;
  switch (phase) {
    case BWD_PREP:
      if constexpr (NORM) {
        hipLaunchKernelGGL((bwd_prep_kernel<T, DV, DVP>), dim3((unsigned)((pa.rows + 3) / 4)), dim3(256), 0, s, pa);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    case BWD_PRE:
      if (a.half0 > 0 && (DK > 64 || a.nseg != 2 || (a.half0 * a.kc) % BC != 0)) return hipErrorInvalidValue;
      hipLaunchKernelGGL((bwd_pre_kernel<T, DK, DV, DVP, BC, NORM, DK <= 64 ? 2 : 1>),
                         dim3(BH * a.nseg + BH * (a.nseg - 1) + (a.half0 > 0 ? BH : 0)),
                         dim3(BWD_PRE_THREADS), 0, s, a);
      return hipGetLastError();
    case BWD_RSCAN:
      hipLaunchKernelGGL((bwd_rscan_kernel<DK, DV, DVP, NORM>), dim3(BH, DK / 16), dim3(256), 0, s, a, gL);
      return hipGetLastError();
    case BWD_WALK:
      hipLaunchKernelGGL((bwd_walk_kernel<T, DK, DV, DVP, BC, NORM>), dim3(BH * a.nseg), dim3(BWD_THREADS), 0, s, a);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK, int DV>
static hipError_t launch_bwd_n(bool norm, int phase, int BH, const BwdArgs &a, const BwdPrepArgs &pa, float gL,
                               hipStream_t s) {
  return norm ? launch_bwd_t<T, DK, DV, true>(phase, BH, a, pa, gL, s)
              : launch_bwd_t<T, DK, DV, false>(phase, BH, a, pa, gL, s);
}

hipError_t launch_bwd(int dtype, int DK, int DV, bool norm, int phase, int BH, const BwdArgs &a,
                      const BwdPrepArgs &pa, float gL, hipStream_t s) {
  if (dtype == 0) {
    if (DK == 16 && DV == 16) return launch_bwd_n<float, 16, 16>(norm, phase, BH, a, pa, gL, s);
    if (DK == 64 && DV == 64) return launch_bwd_n<float, 64, 64>(norm, phase, BH, a, pa, gL, s);
    return hipErrorInvalidValue;
  }
  if (DK == 64 && DV == 64) return launch_bwd_n<bf16, 64, 64>(norm, phase, BH, a, pa, gL, s);
  if (DK == 64 && DV == 128) return launch_bwd_n<bf16, 64, 128>(norm, phase, BH, a, pa, gL, s);
  if (DK == 128 && DV == 64) return launch_bwd_n<bf16, 128, 64>(norm, phase, BH, a, pa, gL, s);
  if (DK == 128 && DV == 128) return launch_bwd_n<bf16, 128, 128>(norm, phase, BH, a, pa, gL, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
