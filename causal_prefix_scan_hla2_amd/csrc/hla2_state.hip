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
//   z = g S q + k (k . q)  (= S_new q),  S <- g S + k k^T,  U <- g^2 U + z v^T,  u <- g^2 u + z,
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

  constexpr int TB = 16;  // tail rows staged at a time
  __shared__ __attribute__((aligned(16))) float sh[DK * DK + DK * DV + 3 * DK];
  __shared__ __attribute__((aligned(16))) T tsh[TB * (2 * DK + DV)];
  float *St = sh;                 // S; it is symmetric, so St[k * DK + i] = S[i][k] as well
  float *Cs = St + DK * DK;       // C rows: Cs[k * DV + j]
  float *ms = Cs + DK * DV;       // m
  float *zv = ms + DK;            // z of a tail token (two buffers)
  T *tq = tsh, *tk = tq + TB * DK, *tvv = tk + TB * DK;  // staged tail rows

  // a sequence shorter than one chunk is all tail: no summary was written (sums is null)
  const float *sums = a.sums ? a.sums + (long)bh * a.nseg * SB : nullptr;
  auto gam_tokens = [&](int t) -> float { return a.decay_on ? exp2f((float)t * a.log2g) : 1.f; };
  const int seg_tokens = a.cps * a.kc;
  const int last_tok0 = L * seg_tokens;
  const int last_full = ((min(a.n, last_tok0 + seg_tokens) - last_tok0) / a.kc) * a.kc;  // tokens in L's summary
  const float GL = gam_tokens(last_full);

  // ---- U, u: combine of the prefix of L with the summary of L (the summary alone when L is the
  // only segment, whose prefix is zero)
  f32x4 U[NBT][4];  // rows i0 + 0..3 of block (i0, j0), columns j0 .. j0+3
  float u = 0.f;    // u[tid] for tid < DK
  const float *pref = a.nseg > 1 ? a.prefix + ((long)bh * a.nseg + L) * PB : nullptr;
#pragma unroll
  for (int b = 0; b < NBT; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) U[b][r] = zero4();
  if (sums) {
    const float *sL = sums + (long)L * SB;
    const float *SL = sL, *CL = SL + DK * DK, *UL = CL + DK * DV, *mL = UL + DK * DV, *uL = mL + DK;
    if (pref) {
      for (int e = tid; e < DK * DK; e += NT) St[e] = pref[e];  // S0
      for (int e = tid; e < DK * DV; e += NT) Cs[e] = CL[e];
      for (int e = tid; e < DK; e += NT) ms[e] = mL[e];
      __syncthreads();
    }
#pragma unroll
    for (int b = 0; b < NBT; ++b) {
      const int blk = tid + b * NT;
      if (blk < NB4) {
        const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
        f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
        if (pref) {
          for (int k = 0; k < DK; ++k) {
            const f32x4 sc = *(const f32x4 *)(St + k * DK + i0);
            const f32x4 cr = *(const f32x4 *)(Cs + k * DV + j0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += sc[r] * cr;
          }
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
      if (pref)
        for (int k = 0; k < DK; ++k) s += St[k * DK + tid] * ms[k];
      const float u0 = pref ? pref[DK * DK + DK * DV + tid] : 0.f;
      u = GL * GL * u0 + uL[tid] + GL * s;
    }
  }
  __syncthreads();

  // ---- S, C, m: fold of every summary (a thread's elements of one summary are loaded together)
  const float Gf = gam_tokens(seg_tokens);
  {
    constexpr int NS = (DK * DK + NT - 1) / NT, NC = (DK * DV + NT - 1) / NT;
    float xs[NS], xc[NC], xm = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) xs[i] = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) xc[i] = 0.f;
    for (int r = 0; sums && r <= L; ++r) {
      const float G = r < L ? Gf : GL;
      const float *sr = sums + (long)r * SB;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = tid + i * NT;
        if (NS * NT == DK * DK || e < DK * DK) xs[i] = G * xs[i] + sr[e];
      }
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int e = tid + i * NT;
        if (NC * NT == DK * DV || e < DK * DV) xc[i] = G * xc[i] + sr[DK * DK + e];
      }
      if (tid < DK) xm = G * xm + sr[DK * DK + 2 * DK * DV + tid];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = tid + i * NT;
      if (NS * NT == DK * DK || e < DK * DK) St[e] = xs[i];
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int e = tid + i * NT;
      if (NC * NT == DK * DV || e < DK * DV) Cs[e] = xc[i];
    }
    if (tid < DK) ms[tid] = xm;
  }
  __syncthreads();

  // ---- the tokens after the last full chunk, in order
  // Their rows are staged TB at a time.  For the tail the state lives in registers: every
  // thread keeps its 4x4 blocks of S and of C (the blocks of U), and m, u for tid < DK.  Per
  // token, z = S_t q_t is formed from the state before the token, z = g S_{t-1} q + k (k . q):
  // each thread's partial sums over its S blocks' columns are reduced across the lanes that
  // share those rows, and z goes through LDS (two buffers, by token parity) to the U blocks.
  // One barrier per token.
  const int tail0 = last_tok0 + last_full;
  if (tail0 < a.n) {
    const float g = a.decay_on ? exp2f(a.log2g) : 1.f, g2 = g * g;
    const T *qh = (const T *)a.q + (long)bh * a.n * d, *kh = (const T *)a.k + (long)bh * a.n * d;
    const T *vh = (const T *)a.v + (long)bh * a.n * dv;
    constexpr int SPR = DK / 4;                        // S blocks per row (lanes that share rows)
    constexpr int NB4S = DK * DK / 16, NBS = (NB4S + NT - 1) / NT;
    static_assert(SPR <= 64 && (SPR & (SPR - 1)) == 0, "S row blocks within a wave");
    f32x4 Sr[NBS][4], Cr[NBT][4];
    float mreg = 0.f;
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int blk = tid + b * NT;
      const int i0 = 4 * (blk / SPR), j0 = 4 * (blk % SPR);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        Sr[b][rr] = (NBS * NT == NB4S || blk < NB4S) ? *(const f32x4 *)(St + (i0 + rr) * DK + j0) : zero4();
    }
#pragma unroll
    for (int b = 0; b < NBT; ++b) {
      const int blk = tid + b * NT;
      const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        Cr[b][rr] = (NBT * NT == NB4 || blk < NB4) ? *(const f32x4 *)(Cs + (i0 + rr) * DV + j0) : zero4();
    }
    if (tid < DK) mreg = ms[tid];
    auto ld4 = [](const T *p) -> f32x4 { return f32x4{(float)p[0], (float)p[1], (float)p[2], (float)p[3]}; };
    int par = 0;
    for (int tb = tail0; tb < a.n; tb += TB) {
      const int nb = min(TB, a.n - tb);
      __syncthreads();  // every read of the previous rows done
      for (int e = tid; e < TB * DK; e += NT) {
        const int r = e / DK, c = e % DK;
        const bool ok = r < nb && c < d;
        tq[e] = ok ? qh[(long)(tb + r) * d + c] : (T)0.f;
        tk[e] = ok ? kh[(long)(tb + r) * d + c] : (T)0.f;
      }
      for (int e = tid; e < TB * DV; e += NT) {
        const int r = e / DV, c = e % DV;
        tvv[e] = (r < nb && c < dv) ? vh[(long)(tb + r) * dv + c] : (T)0.f;
      }
      __syncthreads();
      for (int r = 0; r < nb; ++r, par ^= 1) {
        const T *q = tq + r * DK, *k = tk + r * DK, *v = tvv + r * DV;
        float *const z = zv + par * DK;
        // z from S_{t-1}, then S absorbs the token
#pragma unroll
        for (int b = 0; b < NBS; ++b) {
          const int blk = tid + b * NT;
          const int i0 = 4 * (blk / SPR), j0 = 4 * (blk % SPR);
          const bool own = NBS * NT == NB4S || blk < NB4S;
          const f32x4 qj = ld4(q + j0), kj = ld4(k + j0), ki = ld4(k + i0);
          float zp[4], kq = kj[0] * qj[0] + kj[1] * qj[1] + kj[2] * qj[2] + kj[3] * qj[3];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            zp[rr] = Sr[b][rr][0] * qj[0] + Sr[b][rr][1] * qj[1] + Sr[b][rr][2] * qj[2] + Sr[b][rr][3] * qj[3];
#pragma unroll
          for (int o = 1; o < SPR; o <<= 1) {
            kq += __shfl_xor(kq, o);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) zp[rr] += __shfl_xor(zp[rr], o);
          }
          if (own && j0 == 0) *(f32x4 *)(z + i0) = f32x4{g * zp[0], g * zp[1], g * zp[2], g * zp[3]} + kq * ki;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) Sr[b][rr] = g * Sr[b][rr] + ki[rr] * kj;
        }
        // C, m absorb the token
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
          const int blk = tid + b * NT;
          const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
          const f32x4 qi = ld4(q + i0), vj = ld4(v + j0);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) Cr[b][rr] = g * Cr[b][rr] + qi[rr] * vj;
        }
        if (tid < DK) mreg = g * mreg + (float)q[tid];
        __syncthreads();  // z complete
        // U, u absorb z v^T, z
        if (tid < DK) u = g2 * u + z[tid];
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
          const int blk = tid + b * NT;
          const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
          const f32x4 vj = ld4(v + j0), zi = *(const f32x4 *)(z + i0);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) U[b][rr] = g2 * U[b][rr] + zi[rr] * vj;
        }
      }
    }
    // the state back to LDS for the products below
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int blk = tid + b * NT;
      const int i0 = 4 * (blk / SPR), j0 = 4 * (blk % SPR);
      if (NBS * NT == NB4S || blk < NB4S) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) *(f32x4 *)(St + (i0 + rr) * DK + j0) = Sr[b][rr];
      }
    }
#pragma unroll
    for (int b = 0; b < NBT; ++b) {
      const int blk = tid + b * NT;
      const int i0 = 4 * (blk / BPR), j0 = 4 * (blk % BPR);
      if (NBT * NT == NB4 || blk < NB4) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) *(f32x4 *)(Cs + (i0 + rr) * DV + j0) = Cr[b][rr];
      }
    }
    if (tid < DK) ms[tid] = mreg;
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
  for (int e = tid; e < d * d; e += NT) oS[e] = St[(e / d) * DK + e % d];
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
