// hla2_mfma.h -- gfx950 MFMA fragment helpers shared by the HLA2 kernels.
//
// All matrix products go through one MFMA shape per element type:
//   bf16: v_mfma_f32_16x16x32_bf16 (16x16 output, k-step 32, 8 k-values per lane)
//   f32 : v_mfma_f32_16x16x4f32    (16x16 output, k-step 4,  1 k-value per lane)
// Output (accumulator) layout, both types: lane (g = lane/16, n = lane%16) holds
// rows 4g..4g+3 of column n of the 16x16 tile.
//
// Operand k-order.  A "k-tile" is 32 k-values for bf16 (one MFMA) and 16 for f32
// (four MFMAs).  Within a k-tile starting at k0, lane group g holds the k-values
//   bf16: k0+4g+0..3 (elements 0..3) and k0+16+4g+0..3 (elements 4..7)
//   f32 : k0+4g+s for MFMA step s = 0..3
// This is exactly the row set an accumulator tile pair (bf16) or tile (f32)
// gives a lane, so a product's output can feed the next product's operand from
// registers without passing through LDS.  LDS operands are read in the same
// order: along a row with plain loads, down a column with the gfx950 LDS
// transpose read (ds_read_b64_tr_b16), which hands each lane of a 16-lane group
// one 16-bit element from each of four 4-element rows supplied by its neighbours.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename T> struct Ktile;
template <> struct Ktile<bf16> {
  static constexpr int ROWS = 32;  // k-values per k-tile
  typedef bf16x8 frag;
};
template <> struct Ktile<float> {
  static constexpr int ROWS = 16;
  typedef f32x4 frag;
};

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 MFMA (8 passes) followed by 16 wait states that nothing can be scheduled
// into.  An 8-pass MFMA reads its accumulator input late, so a VALU write to
// that register must wait 7 states; with this compiler the f32 form has been
// seen emitted with a VALU overwrite of its accumulator input right after the
// MFMA (and wrong results).  The explicit gap makes every such write safe.
__device__ __forceinline__ f32x4 mfma_f32_guarded(float a, float b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  return c;
}
__device__ __forceinline__ f32x4 mma(const f32x4 &a, const f32x4 &b, f32x4 c) {
  c = mfma_f32_guarded(a[0], b[0], c);
  c = mfma_f32_guarded(a[1], b[1], c);
  c = mfma_f32_guarded(a[2], b[2], c);
  c = mfma_f32_guarded(a[3], b[3], c);
  return c;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over `bytes` bytes at `base` (gfx9 data format word): loads
// at or past `bytes` return zero and stores there are dropped, so guarded global
// accesses need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
// a byte offset past the end of every buffer resource (sizes stay below 2^31)
constexpr int OOB_OFFSET = 0x7ffffff0;

// Load *p when ok, else zero.  The load itself always reads a valid global
// address (`safe` when !ok) and the zeroing is a select on the value, so the
// compiler never has to give a zero constant an address.
template <typename V>
__device__ __forceinline__ V ld_or_zero(const V *p, const V *safe, bool ok) {
  V x = *(ok ? p : safe);
  return ok ? x : V{};
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---- fragments from rows (k contiguous in memory) --------------------------
// lane (g, n) gets X[row0 + n][k-order of group g]
__device__ __forceinline__ bf16x8 ld_rows(const bf16 *X, int ld, int row0, int k0, int lane) {
  const bf16 *p = X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  return cat8(*(const bf16x4 *)p, *(const bf16x4 *)(p + 16));
}
__device__ __forceinline__ f32x4 ld_rows(const float *X, int ld, int row0, int k0, int lane) {
  return *(const f32x4 *)(X + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
}

// ---- fragments from columns (k strided in memory) --------------------------
// lane (g, n) gets X[k-order of group g][col0 + n]; X must live in LDS.
__device__ __forceinline__ bf16x8 ld_cols(const bf16 *X, int ld, int k0, int col0, int lane) {
  const int g = lane >> 4, src = lane & 15;
  const bf16 *p = X + (k0 + 4 * g + (src >> 2)) * ld + col0 + 4 * (src & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * ld));
  return cat8(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi));
}
__device__ __forceinline__ f32x4 ld_cols(const float *X, int ld, int k0, int col0, int lane) {
  const float *p = X + (k0 + 4 * (lane >> 4)) * ld + col0 + (lane & 15);
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// k-value index (relative to the k-tile start) of element e for lane group g
template <typename T> __device__ __forceinline__ int kidx(int g, int e);
template <> __device__ __forceinline__ int kidx<bf16>(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }
template <> __device__ __forceinline__ int kidx<float>(int g, int e) { return 4 * g + e; }

// scale every element of a fragment by a per-k factor
template <typename F>
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 f, int g, F &&w) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)((float)f[e] * w(kidx<bf16>(g, e)));
  return r;
}
template <typename F>
__device__ __forceinline__ f32x4 scale_frag(f32x4 f, int g, F &&w) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = f[e] * w(kidx<float>(g, e));
  return r;
}

// operand fragment of a k-tile from accumulator tiles (rows 0-15 and, for bf16, 16-31)
__device__ __forceinline__ bf16x8 frag_from_acc(f32x4 t0, f32x4 t1) {
  return bf16x8{(bf16)t0[0], (bf16)t0[1], (bf16)t0[2], (bf16)t0[3],
                (bf16)t1[0], (bf16)t1[1], (bf16)t1[2], (bf16)t1[3]};
}
__device__ __forceinline__ f32x4 frag_from_acc(f32x4 t0) { return t0; }

// store 4 consecutive values of one row (an accumulator's 4 rows seen transposed)
__device__ __forceinline__ void st4(bf16 *p, f32x4 x) {
  *(bf16x4 *)p = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
__device__ __forceinline__ void st4(float *p, f32x4 x) { *(f32x4 *)p = x; }

// sum over the four lane groups (lanes n, n+16, n+32, n+48)
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace hla2
