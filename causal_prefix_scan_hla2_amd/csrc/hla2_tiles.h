// hla2_tiles.h -- generic MFMA tile machinery of the chunk walkers that take
// all their operands from LDS (the backward pass and AHLA): tile products with
// either operand transposed, the split of a result's 16x16 tiles over the
// waves of a workgroup, and row tiles fetched from global memory a chunk ahead.
#pragma once
#include "hla2_mfma.h"

namespace hla2 {

// ---------------------------------------------------------------------------
// LDS row layout.  A bf16 operand fragment takes, per lane group g, the k-values
// 4g..4g+3 and 16+4g..16+4g+3 of a 32-wide k-tile (hla2_mfma.h).  In LDS every
// row keeps its 4-column groups permuted inside each 32 columns so that those two
// groups sit side by side: a row fragment is then one 16-byte read instead of two
// 8-byte reads 32 bytes apart (which the compiler pairs into one slow read).  The
// LDS transpose read still finds any logical 4-column group, since every lane
// supplies its own address.  fp32 rows are stored as they are.
template <typename T> __device__ __forceinline__ int pcol(int c);
template <> __device__ __forceinline__ int pcol<bf16>(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
template <> __device__ __forceinline__ int pcol<float>(int c) { return c; }

// bf16 rows are also swizzled: the 16-byte piece j of row r sits at piece j ^ s(r), with s chosen
// by the row pitch.  LDS cycles per wave-wide access, measured on the device for this layout
// (transpose read / 8-byte accumulator-row write / 16-byte row read / staging write of a row's
// two 4-column groups):
//   pitch = 32 mod 64 bytes (96, 160, 224, 288, 352): no swizzle 4 / 16 / 4 / 16;
//                                                     s = bit 2 of r: 4 / 8 / 4 / 8;
//   pitch = 16 mod 64 bytes (80, 144, 208, 272, 336): no swizzle 6 / 8 / 8 / 8 (8 / 8 / 8 / 8 at 272);
//                                                     s = bit 2 ^ bit 3 of r: 6 / 8 / 4 / 4.
// Only the first kind is swizzled: at the second (the backward's adjoint-summary role, whose 16-byte
// padding lets two workgroups share a CU) s = bit 2 ^ bit 3 measured no faster, and the chunk states
// in global memory keep their plain layout.  tsw is the swizzle's element
// offset; the rows of one access differ in bits 2 and 3 only through the lane, so with the pitch a
// compile-time constant it is a per-lane constant.
template <typename T> __device__ __forceinline__ int tsw(int row, int ld);
template <> __device__ __forceinline__ int tsw<bf16>(int row, int ld) {
  return ((2 * ld) & 63) == 32 ? ((row >> 2) & 1) << 3 : 0;
}
template <> __device__ __forceinline__ int tsw<float>(int, int) { return 0; }

// Row padding in bytes.  bf16 rows 160 or 288 bytes apart (32 bytes of padding on 128- and
// 256-byte rows) serve 16-byte row reads and LDS transpose reads without bank conflicts
// (measured on gfx950); fp32 rows keep 16 bytes.
template <typename T> constexpr int lds_pad_bytes() { return sizeof(T) == 2 ? 32 : 16; }

// fragments of LDS rows / columns in that layout (k0, col0 multiples of the k-tile / 16)
__device__ __forceinline__ bf16x8 ld_rows_l(const bf16 *X, int ld, int row0, int k0, int lane) {
  const int r = row0 + (lane & 15);
  return *(const bf16x8 *)(X + r * ld + k0 + ((8 * (lane >> 4)) ^ tsw<bf16>(r, ld)));
}
__device__ __forceinline__ f32x4 ld_rows_l(const float *X, int ld, int row0, int k0, int lane) {
  return ld_rows(X, ld, row0, k0, lane);
}
__device__ __forceinline__ bf16x8 ld_cols_l(const bf16 *X, int ld, int k0, int col0, int lane) {
  const int g = lane >> 4, src = lane & 15;
  const int r = k0 + 4 * g + (src >> 2);  // and r + 16: the same swizzle
  const bf16 *p = X + r * ld + (pcol<bf16>(col0 + 4 * (src & 3)) ^ tsw<bf16>(r, ld));
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * ld));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}
__device__ __forceinline__ f32x4 ld_cols_l(const float *X, int ld, int k0, int col0, int lane) {
  return ld_cols(X, ld, k0, col0, lane);
}
// four consecutive values of an LDS row at logical column c (a multiple of 4)
template <typename T>
__device__ __forceinline__ void st4l(T *X, int ld, int row, int c, f32x4 x) {
  st4(X + row * ld + (pcol<T>(c) ^ tsw<T>(row, ld)), x);
}

// ---------------------------------------------------------------------------
// Tile products (operands in LDS, in the layout above).  mm: acc(m0.., n0..) += sum_k A(m, k) B(k, n) over k < K, with
// A(m, k) = AT ? A[k*lda + m] : A[m*lda + k] and B(k, n) = BT ? B[n*ldb + k] : B[k*ldb + n].
// Both operands live in LDS (a transposed A or a non-transposed B is read with the
// LDS transpose read).  wk(k) scales the k-th term.
template <bool AT, bool BT, int K, typename T, typename WF>
__device__ __forceinline__ f32x4 mmw(f32x4 acc, const T *A, int lda, const T *B, int ldb, int m0, int n0,
                                     int lane, WF &&wk) {
  constexpr int KT = Ktile<T>::ROWS;
  static_assert(K % KT == 0, "contraction length must be a whole number of k-tiles");
  const int g = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) {
    auto a = AT ? ld_cols_l(A, lda, k0, m0, lane) : ld_rows_l(A, lda, m0, k0, lane);
    auto b = BT ? ld_rows_l(B, ldb, n0, k0, lane) : ld_cols_l(B, ldb, k0, n0, lane);
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
    auto a = AT ? ld_cols_l(A, lda, k0, m0, lane) : ld_rows_l(A, lda, m0, k0, lane);
    auto b = BT ? ld_rows_l(B, ldb, n0, k0, lane) : ld_cols_l(B, ldb, k0, n0, lane);
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
// pt with a causally masked X over the contraction: X(i, k) = 0 for k > i, or with XT (X held as the
// rows of a lower triangle, X(i, k) = L(k, i)) X(i, k) = 0 for k < i.  The tile's rows lie in
// [rlo, rhi + 16); a k-tile that misses the triangle for all of them adds only zeros and is skipped.
// Callers pass bounds that are constants once the tile loop is unrolled (tile_rows_lo / hi), so no
// branch remains.
template <bool XT, bool YT, int K, typename T>
__device__ __forceinline__ f32x4 pt_tri(f32x4 acc, const T *X, int ldx, const T *Y, int ldy, int i0, int j0,
                                        int lane, int rlo, int rhi) {
  constexpr int KT = Ktile<T>::ROWS;
  static_assert(K % KT == 0, "contraction length must be a whole number of k-tiles");
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) {
    if (XT ? k0 + KT <= rlo : k0 >= rhi + 16) continue;
    // as pt: the product is formed transposed, Y's fragment as the A operand
    auto a = YT ? ld_rows_l(Y, ldy, j0, k0, lane) : ld_cols_l(Y, ldy, k0, j0, lane);
    auto b = XT ? ld_cols_l(X, ldx, k0, i0, lane) : ld_rows_l(X, ldx, i0, k0, lane);
    acc = mma(a, b, acc);
  }
  return acc;
}
// the same with weights w(k) on the contraction index: P = X diag(w) Y
template <bool XT, bool YT, int K, typename T, typename WF>
__device__ __forceinline__ f32x4 ptw(f32x4 acc, const T *X, int ldx, const T *Y, int ldy, int i0, int j0, int lane,
                                     WF &&wk) {
  return mmw<!YT, !XT, K>(acc, Y, ldy, X, ldx, j0, i0, lane, wk);
}

// ---------------------------------------------------------------------------
// Two-term operands.  Where one bf16 rounding of an operand costs too much accuracy the
// operand is kept as two bf16 halves, hi = bf16(x) and lo = bf16(x - hi) (about 16
// significant bits), and a product takes one MFMA per half.
// Four values of an LDS row, as one bf16 value (or fp32) or, with SPLIT, as hi and lo halves.
template <bool SPLIT, typename T>
__device__ __forceinline__ void st4_split(T *hi, T *lo, int ld, int row, int c, f32x4 x) {
  if constexpr (SPLIT) {
    f32x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (float)(T)x[e];
    st4l(hi, ld, row, c, h);
    st4l(lo, ld, row, c, x - h);
  } else {
    st4l(hi, ld, row, c, x);
  }
}

// acc + X Y (the pt product), with Y's low half added under SPLIT
template <bool SPLIT, bool XT, bool YT, int K, typename T>
__device__ __forceinline__ f32x4 pt2y(f32x4 acc, const T *X, int ldx, const T *Yh, const T *Yl, int ldy, int i0,
                                      int j0, int lane) {
  acc = pt<XT, YT, K>(acc, X, ldx, Yh, ldy, i0, j0, lane);
  if constexpr (SPLIT) acc = pt<XT, YT, K>(acc, X, ldx, Yl, ldy, i0, j0, lane);
  return acc;
}
// acc + X Y with X's low half added under SPLIT
template <bool SPLIT, bool XT, bool YT, int K, typename T>
__device__ __forceinline__ f32x4 pt2x(f32x4 acc, const T *Xh, const T *Xl, int ldx, const T *Y, int ldy, int i0,
                                      int j0, int lane) {
  acc = pt<XT, YT, K>(acc, Xh, ldx, Y, ldy, i0, j0, lane);
  if constexpr (SPLIT) acc = pt<XT, YT, K>(acc, Xl, ldx, Y, ldy, i0, j0, lane);
  return acc;
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
// The tiles of a BC x BC causally masked product: f(i0, j0, store_ok, live), live false for a tile
// above the diagonal (zero under the mask; the caller skips its products under a wave-uniform branch
// and still stores its zeros).  With 64-token chunks on 8 waves, wave w takes tile w and then tile
// 8 + ((w + 3) & 7), so that the six zero tiles fall 1, 1, 2, 2 on the four SIMDs (waves w and w + 4
// share SIMD w % 4); otherwise the order of for_tiles, where a wave's repeat of the last tile (not
// stored) is not live either.
template <int BC, int NW = BWD_WAVES, typename F>
__device__ __forceinline__ void for_causal_tiles(int w, F &&f) {
  if constexpr (BC == 64 && NW == 8) {
    const int t0 = w, t1 = 8 + ((w + 3) & 7);
    f(16 * (t0 >> 2), 16 * (t0 & 3), true, (t0 & 3) <= (t0 >> 2));
    f(16 * (t1 >> 2), 16 * (t1 & 3), true, (t1 & 3) <= (t1 >> 2));
  } else {
    for_tiles<BC, BC, NW>(w, [&](int i0, int j0, bool ok, int) { f(i0, j0, ok, ok && j0 <= i0); });
  }
}
template <int I, int J, int NW = BWD_WAVES> struct TileCount {
  static constexpr int NT = (I / 16) * (J / 16), PER = (NT + NW - 1) / NW;
};
// First rows of the lowest and highest tile any wave holds at step `it` of for_tiles<I, J, NW>.
template <int I, int J, int NW = BWD_WAVES>
__device__ __forceinline__ constexpr int tile_rows_lo(int it) { return 16 * ((NW * it) / (J / 16)); }
template <int I, int J, int NW = BWD_WAVES>
__device__ __forceinline__ constexpr int tile_rows_hi(int it) {
  constexpr int NT = (I / 16) * (J / 16);
  return 16 * ((NW * it + NW - 1 < NT ? NW * it + NW - 1 : NT - 1) / (J / 16));
}

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
  // into the LDS row layout above: a bf16 vector's two 4-column groups go to their own places
  __device__ __forceinline__ void put(T *dst, int ld, int tid) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NTH;
      if (EVEN || i < TOT) {
        T *row = dst + (i / PERROW) * ld;
        const int c = (i % PERROW) * VN, sw = tsw<T>(i / PERROW, ld);
        if constexpr (VN == 8) {
          *(bf16x4 *)(row + (pcol<T>(c) ^ sw)) = bf16x4{x[j][0], x[j][1], x[j][2], x[j][3]};
          *(bf16x4 *)(row + (pcol<T>(c + 4) ^ sw)) = bf16x4{x[j][4], x[j][5], x[j][6], x[j][7]};
        } else {
          *(V *)(row + c) = x[j];
        }
      }
    }
  }
  // put with row r scaled by exp2(r * log2w) (a token weight g^r); the weight is formed from the
  // row index, so it needs no table in LDS
  __device__ __forceinline__ void put_scaled(T *dst, int ld, int tid, float log2w) const {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * NTH;
      if (EVEN || i < TOT) {
        const int r = i / PERROW, c = (i % PERROW) * VN, sw = tsw<T>(r, ld);
        T *row = dst + r * ld;
        const float wr = exp2f((float)r * log2w);
        V y;
#pragma unroll
        for (int e = 0; e < VN; ++e) y[e] = (T)((float)x[j][e] * wr);
        if constexpr (VN == 8) {
          *(bf16x4 *)(row + (pcol<T>(c) ^ sw)) = bf16x4{y[0], y[1], y[2], y[3]};
          *(bf16x4 *)(row + (pcol<T>(c + 4) ^ sw)) = bf16x4{y[4], y[5], y[6], y[7]};
        } else {
          *(V *)(row + c) = y;
        }
      }
    }
  }
};

// Tile of P = X Y where Y is symmetric or given as its transposed rows: the
// fragments yf[k] = rows j0 .. j0+15 of Y^T over the k-tiles of the contraction
// (read ahead by the caller), X row-major in LDS.  Lane (g, n) holds P[i0 + n][j0 + 4g + e].
template <int K, typename T, typename FR>
__device__ __forceinline__ f32x4 pt_frags(f32x4 acc, const FR *yf, const T *X, int ldx, int i0, int lane) {
  constexpr int KT = Ktile<T>::ROWS;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += KT) acc = mma(yf[k0 / KT], ld_rows_l(X, ldx, i0, k0, lane), acc);
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
