// hla2_state.hip -- the final state of a forward pass, in the decode layout
// S | C | m | G | h, so that streaming decode can continue where the forward
// stopped (technical summary of arXiv 2510.27258 on gist.science, §1 state
// upkeep, and §4: the inclusive scan total is the state after the sequence).
//
// Inputs, per (b, h): the summaries (S_r, C_r, U_r, m_r, u_r) of every segment,
// the last one over its full chunks only; the exclusive prefix (S0, U0, u0) of
// the last segment L; and the tokens after the last full chunk.  With Gamma_r
// = decay^(tokens summarised in segment r):
//   S, C, m  = fold over r of  X <- Gamma_r X + X_r            (elementwise)
//   U        = Gamma_L^2 U0 + U_L + Gamma_L S0 C_L              (the combine of
//   u        = Gamma_L^2 u0 + u_L + Gamma_L S0 m_L               prefix and L)
// then each remaining token (q, k, v) is absorbed in order:
//   S <- g S + k k^T,  z = S q,  U <- g^2 U + z v^T,  u <- g^2 u + z,
//   C <- g C + q v^T,  m <- g m + q
// and finally G = S C - U, h = S m - u.  Everything here is fp32.
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256) state_kernel(StateArgs a) {
  constexpr int NT = 256;
  constexpr int NB4 = DK * DV / 16;                 // 4x4 blocks of a DK x DV matrix
  constexpr int NBT = (NB4 + NT - 1) / NT;          // blocks per thread
  constexpr int BPR = DV / 4;                       // blocks per row
  const long SB = sum_block_floats(DK, DV), PB = prefix_block_floats(DK, DV);
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int d = a.d, dv = a.dv;
  const int L = a.nseg - 1;

  __shared__ __attribute__((aligned(16))) float sh[DK * DK + DK * DV + 4 * DK + DV];
  float *St = sh;                 // S transposed: St[k * DK + i] = S[i][k]
  float *Cs = St + DK * DK;       // C rows: Cs[k * DV + j]
  float *vec = Cs + DK * DV;      // m | u-scratch | q | k | v | z
  float *ms = vec, *qv = ms + DK, *kv = qv + DK, *zv = kv + DK, *vv = zv + DK;

  const float *sums = a.sums + (long)bh * a.nseg * SB;
  auto gam_tokens = [&](int t) -> float { return a.decay_on ? exp2f((float)t * a.log2g) : 1.f; };
  const int seg_tokens = a.cps * a.kc;
  const int last_tok0 = L * seg_tokens;
  const int last_full = ((min(a.n, last_tok0 + seg_tokens) - last_tok0) / a.kc) * a.kc;  // tokens in L's summary
  const float GL = gam_tokens(last_full);

  // ---- U, u: combine of the prefix of L with the summary of L
  const float *sL = sums + (long)L * SB;
  const float *SL = sL, *CL = SL + DK * DK, *UL = CL + DK * DV, *mL = UL + DK * DV, *uL = mL + DK;
  const float *pref = a.nseg > 1 ? a.prefix + ((long)bh * a.nseg + L) * PB : nullptr;
  for (int e = tid; e < DK * DK; e += NT) St[(e % DK) * DK + e / DK] = pref ? pref[e] : 0.f;  // S0^T
  for (int e = tid; e < DK * DV; e += NT) Cs[e] = CL[e];
  for (int e = tid; e < DK; e += NT) ms[e] = mL[e];
  __syncthreads();
  f32x4 U[NBT][4];  // rows i0 + 0..3 of block (i0, j0), columns j0 .. j0+3
  float u = 0.f;    // u[tid] for tid < DK
#pragma unroll
  for (int b = 0; b < NBT; ++b) {
    const int blk = tid + b * NT;
    if (blk < NB4) {
      const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
      f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
      for (int k = 0; k < DK; ++k) {
        const f32x4 sc = *(const f32x4 *)(St + k * DK + i0);
        const f32x4 cr = *(const f32x4 *)(Cs + k * DV + j0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += sc[r] * cr;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 u0 = pref ? *(const f32x4 *)(pref + DK * DK + (i0 + r) * DV + j0) : zero4();
        const f32x4 ul = *(const f32x4 *)(UL + (i0 + r) * DV + j0);
        U[b][r] = GL * GL * u0 + ul + GL * acc[r];
      }
    }
  }
  if (tid < DK) {
    float s = 0.f;
    for (int k = 0; k < DK; ++k) s += St[k * DK + tid] * ms[k];
    const float u0 = pref ? pref[DK * DK + DK * DV + tid] : 0.f;
    u = GL * GL * u0 + uL[tid] + GL * s;
  }
  __syncthreads();

  // ---- S, C, m: fold of every summary
  const float Gf = gam_tokens(seg_tokens);
  for (int e = tid; e < DK * DK; e += NT) {
    float x = 0.f;
    for (int r = 0; r <= L; ++r) x = (r < L ? Gf : GL) * x + sums[(long)r * SB + e];
    St[(e % DK) * DK + e / DK] = x;
  }
  for (int e = tid; e < DK * DV; e += NT) {
    float x = 0.f;
    for (int r = 0; r <= L; ++r) x = (r < L ? Gf : GL) * x + sums[(long)r * SB + DK * DK + e];
    Cs[e] = x;
  }
  for (int e = tid; e < DK; e += NT) {
    float x = 0.f;
    for (int r = 0; r <= L; ++r) x = (r < L ? Gf : GL) * x + sums[(long)r * SB + DK * DK + 2 * DK * DV + e];
    ms[e] = x;
  }
  __syncthreads();

  // ---- the tokens after the last full chunk, in order
  const float g = a.decay_on ? exp2f(a.log2g) : 1.f, g2 = g * g;
  const T *qh = (const T *)a.q + (long)bh * a.n * d, *kh = (const T *)a.k + (long)bh * a.n * d;
  const T *vh = (const T *)a.v + (long)bh * a.n * dv;
  for (int t = last_tok0 + last_full; t < a.n; ++t) {
    for (int e = tid; e < DK; e += NT) {
      qv[e] = e < d ? (float)qh[(long)t * d + e] : 0.f;
      kv[e] = e < d ? (float)kh[(long)t * d + e] : 0.f;
    }
    for (int e = tid; e < DV; e += NT) vv[e] = e < dv ? (float)vh[(long)t * dv + e] : 0.f;
    __syncthreads();
    for (int e = tid; e < DK * DK; e += NT) St[e] = g * St[e] + kv[e / DK] * kv[e % DK];
    for (int e = tid; e < DK * DV; e += NT) Cs[e] = g * Cs[e] + qv[e / DV] * vv[e % DV];
    for (int e = tid; e < DK; e += NT) ms[e] = g * ms[e] + qv[e];
    __syncthreads();
    if (tid < DK) {
      float s = 0.f;
      for (int k = 0; k < DK; ++k) s += St[k * DK + tid] * qv[k];
      zv[tid] = s;
      u = g2 * u + s;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NBT; ++b) {
      const int blk = tid + b * NT;
      if (blk < NB4) {
        const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
        const f32x4 vj = *(const f32x4 *)(vv + j0);
#pragma unroll
        for (int r = 0; r < 4; ++r) U[b][r] = g2 * U[b][r] + zv[i0 + r] * vj;
      }
    }
    __syncthreads();
  }

  // ---- G = S C - U, h = S m - u, and the decode-layout block (actual d, dv)
  float *out = a.state_out + (long)bh * ((long)d * d + 2L * d * dv + 2L * d);
  float *oS = out, *oC = oS + d * d, *om = oC + d * dv, *oG = om + d, *oh = oG + d * dv;
#pragma unroll
  for (int b = 0; b < NBT; ++b) {
    const int blk = tid + b * NT;
    if (blk < NB4) {
      const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
      f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
      for (int k = 0; k < DK; ++k) {
        const f32x4 sc = *(const f32x4 *)(St + k * DK + i0);
        const f32x4 cr = *(const f32x4 *)(Cs + k * DV + j0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += sc[r] * cr;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (i0 + r < d && j0 + c < dv) oG[(i0 + r) * dv + j0 + c] = acc[r][c] - U[b][r][c];
    }
  }
  if (tid < d) {
    float s = 0.f;
    for (int k = 0; k < DK; ++k) s += St[k * DK + tid] * ms[k];
    oh[tid] = s - u;
    om[tid] = ms[tid];
  }
  for (int e = tid; e < d * d; e += NT) oS[e] = St[(e % d) * DK + e / d];
  for (int e = tid; e < d * dv; e += NT) oC[e] = Cs[(e / dv) * DV + e % dv];
}

template <typename T, int DK, int DV>
static hipError_t launch_state_t(int BH, const StateArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((state_kernel<T, DK, DV>), dim3(BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_state(int dtype, int DK, int DV, int BH, const StateArgs &a, hipStream_t s) {
  if (dtype == 0) {
    if (DK == 16 && DV == 16) return launch_state_t<float, 16, 16>(BH, a, s);
    if (DK == 64 && DV == 64) return launch_state_t<float, 64, 64>(BH, a, s);
    return hipErrorInvalidValue;
  }
  if (DK == 64 && DV == 64) return launch_state_t<bf16, 64, 64>(BH, a, s);
  if (DK == 64 && DV == 128) return launch_state_t<bf16, 64, 128>(BH, a, s);
  if (DK == 128 && DV == 64) return launch_state_t<bf16, 128, 64>(BH, a, s);
  if (DK == 128 && DV == 128) return launch_state_t<bf16, 128, 128>(BH, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
