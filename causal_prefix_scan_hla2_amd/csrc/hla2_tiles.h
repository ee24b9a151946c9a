// hla2_tiles.h -- generic MFMA tile machinery of the chunk walkers that take
// all their operands from LDS (the backward pass and AHLA): tile products with
// either operand transposed, the split of a result's 16x16 tiles over the
// waves of a workgroup, and row tiles fetched from global memory a chunk ahead.
#pragma once
#include "hla2_mfma.h"

namespace hla2 {

// ---------------------------------------------------------------------------
// Tile products.  mm: acc(m0.., n0..) += sum_k A(m, k) B(k, n) over k < K, with
// A(m, k) = AT ? A[k*lda + m] : A[m*lda + k] and B(k, n) = BT ? B[n*ldb + k] : B[k*ldb + n].
// A transposed A or a non-transposed B is read with the LDS transpose read, so
// those operands must live in LDS; the others may be global.  wk(k) scales the
// k-th term.
template <bool AT, bool BT, int K, typename T, typename WF>
__device__ __forceinline__ f32x4 mmw(f32x4 acc, const T *A, int lda, const T *B, int ldb, int m0, int n0,
                                     int lane, WF &&wk) {
  constexpr int KT = Ktile<T>::ROWS;
  static_assert(K % KT == 0, "contraction length must be a whole number of k-tiles");
  const int g = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) {
    auto a = AT ? ld_cols(A, lda, k0, m0, lane) : ld_rows(A, lda, m0, k0, lane);
    auto b = BT ? ld_rows(B, ldb, n0, k0, lane) : ld_cols(B, ldb, k0, n0, lane);
    a = scale_frag(a, g, [&](int kk) { return wk(k0 + kk); });
    acc = mma(a, b, acc);
  }
  return acc;
}
template <bool AT, bool BT, int K, typename T>
__device__ __forceinline__ f32x4 mm(f32x4 acc, const T *A, int lda, const T *B, int ldb, int m0, int n0,
                                    int lane) {
  constexpr int KT = Ktile<T>::ROWS;
  static_assert(K % KT == 0, "contraction length must be a whole number of k-tiles");
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) {
    auto a = AT ? ld_cols(A, lda, k0, m0, lane) : ld_rows(A, lda, m0, k0, lane);
    auto b = BT ? ld_rows(B, ldb, n0, k0, lane) : ld_cols(B, ldb, k0, n0, lane);
    acc = mma(a, b, acc);
  }
  return acc;
}
// Tile of P = X Y at P-rows i0.., P-columns j0.., computed as P^T so that lane
// (g, n) holds P[i0 + n][j0 + 4g + e], e = 0..3.  XT: X(i, k) stored at X[k*ldx + i];
// YT: Y(k, j) stored at Y[j*ldy + k].
template <bool XT, bool YT, int K, typename T>
__device__ __forceinline__ f32x4 pt(f32x4 acc, const T *X, int ldx, const T *Y, int ldy, int i0, int j0, int lane) {
  return mm<!YT, !XT, K>(acc, Y, ldy, X, ldx, j0, i0, lane);
}
// the same with weights w(k) on the contraction index: P = X diag(w) Y
template <bool XT, bool YT, int K, typename T, typename WF>
__device__ __forceinline__ f32x4 ptw(f32x4 acc, const T *X, int ldx, const T *Y, int ldy, int i0, int j0, int lane,
                                     WF &&wk) {
  return mmw<!YT, !XT, K>(acc, Y, ldy, X, ldx, j0, i0, lane, wk);
}

// Waves per workgroup of these walkers (two per SIMD).
constexpr int BWD_WAVES = 8, BWD_THREADS = 64 * BWD_WAVES;

// Iterate a wave's share of the 16x16 tiles of an I x J result over NW waves:
// f(i0, j0, store_ok, slot).  A wave with no tile left repeats the last one (not stored).
// When the waves divide the tiles evenly (w < NW), every tile is real and store_ok is
// a compile-time true: no branch around the stores.
template <int I, int J, int NW = BWD_WAVES, typename F>
__device__ __forceinline__ void for_tiles(int w, F &&f) {
  constexpr int NJ = J / 16, NT = (I / 16) * NJ, PER = (NT + NW - 1) / NW;
  constexpr bool EVEN = NT % NW == 0;
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int t = w + NW * it;
    const int tt = (EVEN || t < NT) ? t : NT - 1;
    f(16 * (tt / NJ), 16 * (tt % NJ), EVEN || t < NT, it);
  }
}
template <int I, int J, int NW = BWD_WAVES> struct TileCount {
  static constexpr int NT = (I / 16) * (J / 16), PER = (NT + NW - 1) / NW;
};

// 16-byte vector of the element type
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  typedef bf16x8 type;
  static constexpr int N = 8;
};
template <> struct Vec16<float> {
  typedef f32x4 type;
  static constexpr int N = 4;
};

// Rows [t0, t0+BC) of one head's [n][gc] global matrix at `src`, as LDS rows of
// width W (zero past n and past column gc; with ones >= 0, column `ones` holds 1
// for rows before n).  fetch() reads a thread's share into registers with buffer
// loads (reads past the head's rows return zero, so no branch), put() writes them
// to LDS, so the global reads of the next chunk can fly during this one.
template <typename T, int BC, int W, int NTH = BWD_THREADS>
struct RowTile {
  typedef typename Vec16<T>::type V;
  static constexpr int VN = Vec16<T>::N, PERROW = W / VN, TOT = BC * PERROW, PER = (TOT + NTH - 1) / NTH;
  static constexpr bool EVEN = TOT % NTH == 0;  // every thread has PER vectors: no guard
  V x[PER];
  __device__ __forceinline__ void fetch(const T *src, int gc, int t0, int n, int ones, int tid) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src, n * gc * (int)sizeof(T));
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NTH;
      const int r = i / PERROW, c = (i % PERROW) * VN, t = t0 + r;
      const bool in = EVEN || i < TOT;
      int off = (in && c < gc) ? (t * gc + c) * (int)sizeof(T) : OOB_OFFSET;
      asm("" : "+v"(off));  // one load of a selected offset, not a load on each side of a branch
      V v = __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      if (in && c == ones && t < n) v[0] = (T)1.f;
      x[j] = v;
    }
  }
  __device__ __forceinline__ void put(T *dst, int ld, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NTH;
      if (EVEN || i < TOT) *(V *)(dst + (i / PERROW) * ld + (i % PERROW) * VN) = x[j];
    }
  }
};

// Tile of P = X Y where Y is symmetric or given as its transposed rows: the
// fragments yf[k] = rows j0 .. j0+15 of Y^T over the k-tiles of the contraction
// (read ahead by the caller), X row-major.  Lane (g, n) holds P[i0 + n][j0 + 4g + e].
template <int K, typename T, typename FR>
__device__ __forceinline__ f32x4 pt_frags(f32x4 acc, const FR *yf, const T *X, int ldx, int i0, int lane) {
  constexpr int KT = Ktile<T>::ROWS;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) acc = mma(yf[k0 / KT], ld_rows(X, ldx, i0, k0, lane), acc);
  return acc;
}

// Store four consecutive values of row t, columns c .. c+3, of one head's [n][ncols]
// matrix at `base` with a buffer store: rows past n and columns past ncols are dropped.
__device__ __forceinline__ void st_out(bf16 *base, int ncols, int t, int c, int n, f32x4 x) {
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(base, n * ncols * 2);
  const bf16x4 b = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), r, c < ncols ? (t * ncols + c) * 2 : OOB_OFFSET,
                                        0, 0);
}
__device__ __forceinline__ void st_out(float *base, int ncols, int t, int c, int n, f32x4 x) {
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(base, n * ncols * 4);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, c < ncols ? (t * ncols + c) * 4 : OOB_OFFSET,
                                         0, 0);
}
__device__ __forceinline__ void st4g(bf16 *p, f32x4 x) { *(bf16x4 *)p = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]}; }
__device__ __forceinline__ void st4g(float *p, f32x4 x) { *(f32x4 *)p = x; }

}  // namespace hla2
