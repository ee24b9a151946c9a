// hla2_decode.hip -- fused single-token streaming step, state updated in place.
//
// Technical summary of arXiv 2510.27258 (gist.science), §1: the per-head state
// is the prefix summaries S (key moment), C (query-value accumulator), m
// (query mass) and the cross summaries G, h; one token costs O(d^2 + d dv)
// independent of the position.  With decay g, for token (q, k, v):
//   G <- g^2 G + g k (k^T C_old),   h <- g^2 h + g k (k^T m_old)
//   S <- g S + k k^T,   C <- g C + q v^T,   m <- g m + q
//   num = q^T (S C - G) = p^T C - q^T G  with p = S q (S symmetric)
//   den = q^T (S m - h) = p . m - q . h
// Expanded so every state matrix is streamed through registers exactly once:
//   p      = g (S_old q) + (q.k) k
//   q^T G  = g^2 (q^T G_old) + g (q.k) (k^T C_old)
// One workgroup (256 threads) owns one (sequence, head) block; each thread owns
// 4 consecutive columns of a strip of rows, so every row is read and written
// with coalesced 16-byte accesses.  The state is HBM-resident and touched once
// per step (read + write), which is the whole cost of the step.  Its loads and
// stores are non-temporal: no block is touched again within a step, so keeping
// it in the caches only evicts other blocks' lines (measured on the 256 x 32
// head, d = dv = 64 workload: 154 -> 142 us per step).
#include "hla2_internal.h"
#include "hla2_mfma.h"

namespace hla2 {

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

template <typename T, int D, int DV>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr long L = (long)D * D + 2L * D * DV + 2L * D;
  // thread -> (row offset, column group) for rows of length D (S) and DV (C, G)
  constexpr int TS = D / 4, RS = 256 / TS, NS = (D + RS - 1) / RS;
  constexpr int TV = DV / 4, RV = 256 / TV, NV = (D + RV - 1) / RV;
  constexpr int RMAX = RS > RV ? RS : RV;

  __shared__ float qs[D], ks[D], vs[DV], ps[D], ms[D], hs[D];
  __shared__ float red[3][RMAX][DV > D ? DV : D];
  __shared__ float scal[4];

  const int tid = threadIdx.x;
  const long bh = blockIdx.x;
  float *st = a.state + bh * L;
  float *S = st, *C = S + D * D, *m = C + D * DV, *G = m + D, *h = G + D * DV;
  const float gam = a.gamma, g2 = a.gamma * a.gamma;

  // ---- issue every state load first
  const int sc = tid % TS, sr0 = tid / TS;
  const int vc = tid % TV, vr0 = tid / TV;
  f32x4 Sr[NS], Cr[NV], Gr[NV];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = sr0 + i * RS;
    Sr[i] = r < D ? __builtin_nontemporal_load((const f32x4 *)(S + r * D + 4 * sc)) : zero4();
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int r = vr0 + i * RV;
    Cr[i] = r < D ? __builtin_nontemporal_load((const f32x4 *)(C + r * DV + 4 * vc)) : zero4();
    Gr[i] = r < D ? __builtin_nontemporal_load((const f32x4 *)(G + r * DV + 4 * vc)) : zero4();
  }
  if (tid < D) {
    qs[tid] = to_f(((const T *)a.q)[bh * D + tid]);
    ks[tid] = to_f(((const T *)a.k)[bh * D + tid]);
    ms[tid] = m[tid];
    hs[tid] = h[tid];
  }
  if (tid < DV) vs[tid] = to_f(((const T *)a.v)[bh * DV + tid]);
  __syncthreads();

  // ---- pass 1: partial sums of S_old^T q, k^T C_old, q^T G_old; write S, C updates
  float pq[4] = {0, 0, 0, 0}, pk[4] = {0, 0, 0, 0}, pg[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int r = sr0 + i * RS;
    if (r < D) {
      const float qr = qs[r], kr = ks[r];
      f32x4 nw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pq[e] += qr * Sr[i][e];
        nw[e] = gam * Sr[i][e] + kr * ks[4 * sc + e];
      }
      __builtin_nontemporal_store(nw, (f32x4 *)(S + r * D + 4 * sc));
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int r = vr0 + i * RV;
    if (r < D) {
      const float qr = qs[r], kr = ks[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pk[e] += kr * Cr[i][e];
        pg[e] += qr * Gr[i][e];
        Cr[i][e] = gam * Cr[i][e] + qr * vs[4 * vc + e];  // C_new kept for the readout
      }
      __builtin_nontemporal_store(Cr[i], (f32x4 *)(C + r * DV + 4 * vc));
    }
  }
  if (sr0 < RS) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[0][sr0][4 * sc + e] = pq[e];
  }
  if (vr0 < RV) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      red[1][vr0][4 * vc + e] = pk[e];
      red[2][vr0][4 * vc + e] = pg[e];
    }
  }
  if (tid < 64) {  // q.k and k.m_old
    float qk = 0.f, km = 0.f;
    for (int x = tid; x < D; x += 64) {
      qk += qs[x] * ks[x];
      km += ks[x] * ms[x];
    }
    for (int o = 32; o >= 1; o >>= 1) {
      qk += __shfl_xor(qk, o);
      km += __shfl_xor(km, o);
    }
    if (tid == 0) {
      scal[0] = qk;
      scal[1] = km;
    }
  }
  __syncthreads();
  const float qk = scal[0], km = scal[1];
  // reduce partials: p (length D) and kC, qG (length DV)
  if (tid < D) {
    float s = 0.f;
    for (int r = 0; r < (RS < D ? RS : D); ++r) s += red[0][r][tid];
    ps[tid] = gam * s + qk * ks[tid];
  }
  float kC = 0.f, qG = 0.f;
  const int rv_used = RV < D ? RV : D;
  // every thread needs kC for its own 4 columns; thread tid < DV also finishes qG
  __syncthreads();
  float kc4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s = 0.f;
    for (int r = 0; r < rv_used; ++r) s += red[1][r][4 * vc + e];
    kc4[e] = s;
  }
  if (tid < DV) {
    for (int r = 0; r < rv_used; ++r) {
      kC += red[1][r][tid];
      qG += red[2][r][tid];
    }
  }

  // ---- pass 2: G update and the readout partials p^T C_new
  float pc[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int r = vr0 + i * RV;
    if (r < D) {
      const float kr = ks[r], pr = ps[r];
      f32x4 nw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nw[e] = g2 * Gr[i][e] + gam * kr * kc4[e];
        pc[e] += pr * Cr[i][e];
      }
      __builtin_nontemporal_store(nw, (f32x4 *)(G + r * DV + 4 * vc));
    }
  }
  // m, h updates and the denominator
  if (tid < D) {
    const float mn = gam * ms[tid] + qs[tid];
    const float hn = g2 * hs[tid] + gam * ks[tid] * km;
    m[tid] = mn;
    h[tid] = hn;
    ms[tid] = ps[tid] * mn - qs[tid] * hn;  // per-row term of den
  }
  __syncthreads();
  if (vr0 < RV) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[0][vr0][4 * vc + e] = pc[e];
  }
  if (tid < 64) {
    float dsum = 0.f;
    for (int x = tid; x < D; x += 64) dsum += ms[x];
    for (int o = 32; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o);
    if (tid == 0) scal[2] = dsum;
  }
  __syncthreads();
  if (tid < DV) {
    float s = 0.f;
    for (int r = 0; r < rv_used; ++r) s += red[0][r][tid];
    const float num = s - (g2 * qG + gam * qk * kC);
    const float o = a.normalize ? num / scal[2] : num;
    ((T *)a.out)[bh * DV + tid] = (T)o;
  }
}

template <typename T>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
#define HLA2_DEC(D_, DV_)                                                                    \
  if (a.d == D_ && a.dv == DV_) {                                                            \
    hipLaunchKernelGGL((decode_kernel<T, D_, DV_>), dim3(a.NH), dim3(256), 0, s, a);         \
    return hipGetLastError();                                                                \
  }
  HLA2_DEC(16, 16) HLA2_DEC(16, 32) HLA2_DEC(16, 64) HLA2_DEC(16, 128)
  HLA2_DEC(32, 16) HLA2_DEC(32, 32) HLA2_DEC(32, 64) HLA2_DEC(32, 128)
  HLA2_DEC(64, 16) HLA2_DEC(64, 32) HLA2_DEC(64, 64) HLA2_DEC(64, 128)
  HLA2_DEC(128, 16) HLA2_DEC(128, 32) HLA2_DEC(128, 64) HLA2_DEC(128, 128)
#undef HLA2_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s) {
  return dtype == 0 ? launch_decode_t<float>(a, s) : launch_decode_t<bf16>(a, s);
}

}  // namespace hla2
