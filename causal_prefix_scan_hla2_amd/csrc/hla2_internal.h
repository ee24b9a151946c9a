// hla2_internal.h -- kernel argument blocks and launchers shared by the host
// API (hla2_api.cpp) and the kernel translation units.  Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>

namespace hla2 {

// Arguments of the chunk walker (segment summary and output modes).
struct WalkArgs {
  const void *q, *k, *v;  // [BH, n, d], [BH, n, d], [BH, n, dv]
  void *out;              // [BH, n, dv]           (output mode)
  float *den_out;         // [BH, n] or null        (output mode)
  const float *prefix;    // [BH, nseg] prefix blocks (output mode; null when nseg == 1)
  float *sums;            // [BH, nseg-1] summary blocks (summary mode)
  int n, d, dv, chunk, cps, nseg;
  float log2g;            // log2(decay)
  int decay_on;           // decay < 1
  int normalize;
  int need_den;           // normalize || den_out: carry u (and m)
  int sum_all;            // summary mode: summarise every segment, the last one over its full
                          // chunks only (for the final state); else segments 0 .. nseg-2
  int cps0 = 0;           // chunks of segment 0 (0: cps, like every other segment)
  int seg_lo = 0;         // the launch walks segments seg_lo .. (nseg or nsum) - 1 of every head
  int nbh = 0;            // heads B*H (lead launch: its first nbh workgroups walk segment 0)
  float *prefix_out = nullptr;  // lead launch: the prefix blocks (the buffer `prefix` names), where
                                // segment 0's walk writes the prefix of segment 1
  int pfold = 0;          // output launch of a three-segment lead plan without a scan launch:
                          // segment 2 folds segment 1's summary onto segment 1's prefix itself
  float gamma_seg = 1.f;  // decay^(tokens per full segment), for pfold
};
// summary blocks per (b, h) in the workspace
__host__ __device__ inline int walk_nsum(const WalkArgs &a) { return a.sum_all ? a.nseg : a.nseg - 1; }
// Segment geometry in chunks: segment 0 holds cps0 chunks, every later one cps (the
// last may be shorter).
__host__ __device__ inline int walk_cps0(const WalkArgs &a) { return a.cps0 > 0 ? a.cps0 : a.cps; }
__host__ __device__ inline int walk_seg_chunk0(const WalkArgs &a, int s) {
  return s == 0 ? 0 : walk_cps0(a) + (s - 1) * a.cps;
}
__host__ __device__ inline int walk_seg_chunks(const WalkArgs &a, int s) { return s == 0 ? walk_cps0(a) : a.cps; }

// Arguments of the segment-level exclusive scan.
struct ScanArgs {
  float *sums;        // [BH, nsum] summary blocks (the first nseg-1 are scanned; the parallel
                      // form overwrites U and u of the scanned blocks with its cross terms)
  int nsum;
  float *prefix;      // [BH, nseg] prefix blocks
  int nseg;
  float gamma_seg;    // decay^(tokens per full segment): segments first .. nseg-2 are full
  int first = 0;      // 0: start from the zero state; 1: the prefix of segment 1 is given
                      // (written by segment 0's output walk) and the fold starts there
  int pnseg = 0;      // prefix blocks per head in `prefix` (0: nseg)
  int pmin = 0;       // the prefixes of segments pmin .. nseg-1 are written, the one of segment r
  int pshift = 0;     //   at block r - pshift (bf16 path)
};

// Per-(b,h,segment) block sizes in floats, for padded dims DK, DV.
//   summary block: S[DK*DK] | C[DK*DV] | U[DK*DV] | m[DK] | u[DK]
//   prefix block:  S0[DK*DK] | U0[DK*DV] | u0[DK]
__host__ __device__ inline long sum_block_floats(int DK, int DV) { return (long)DK * DK + 2L * DK * DV + 2L * DK; }
__host__ __device__ inline long prefix_block_floats(int DK, int DV) { return (long)DK * DK + (long)DK * DV + DK; }

// LDS bytes of a chunk-walker instantiation (element size esize, padded
// head dims DK, DV, chunk tile CP; out = output mode).  Shared by the kernel's
// static layout and the host's occupancy estimate.
__host__ __device__ constexpr int walk_lds_bytes(int esize, int DK, int DV, int CP, bool out) {
  const int pade = 16 / esize;
  const int ldk = DK + pade, ldv = DV + pade, ldz = CP + pade;
  const int kz = CP * ldk > DK * ldz ? CP * ldk : DK * ldz;
  const int elems = kz + CP * ldv + DK * ldk + (out ? DV * ldk : 0) + (out ? 0 : CP * ldk);
  return elems * esize + (2 * CP + 1 + DK) * 4;
}
__host__ __device__ constexpr int walk_waves(int CP) { return CP / 16 > 4 ? CP / 16 : 4; }
// workgroups of the walker that fit one CU: LDS-limited, and at most 8 waves
__host__ __device__ constexpr int walk_groups_per_cu(int esize, int DK, int DV, int CP, bool out) {
  const int by_lds = (160 * 1024) / walk_lds_bytes(esize, DK, DV, CP, out);
  const int by_waves = 8 / walk_waves(CP);
  const int gmin = by_lds < by_waves ? by_lds : by_waves;
  return gmin < 1 ? 1 : gmin;
}
// waves each SIMD must hold (the register budget the compiler targets)
__host__ __device__ constexpr int walk_waves_per_eu(int esize, int DK, int DV, int CP, bool out) {
  const int w = walk_groups_per_cu(esize, DK, DV, CP, out) * walk_waves(CP) / 4;
  return w < 1 ? 1 : (w > 2 ? 2 : w);
}

// The 8-wave bf16 walker (hla2_walk8.h): 64-token chunks.  LDS elements (bf16) of an
// instantiation: two Q buffers in output mode (one in summary mode), K, V, Z~ and bf16 S0 rows,
// plus Z and W rows in output mode (and at d <= 64 the staged output rows), each row padded; then
// (bytes) u0 twice, the decay table and
// the two halves' den parts.  One workgroup per CU (eight waves, two per SIMD).
__host__ __device__ constexpr int walk8_lds_elems(int DK, int DV, bool out) {
  const int CP = 64, ldk = DK + 16, ldq = out ? DK + 8 : DK + 16, ldt = DK + 16, lds0 = DK + 16, ldz = DK + 16;
  const int ldv = DV + 16, ldw = CP + 16;
  return (out ? 2 : 1) * CP * ldq + CP * ldk + CP * ldv + CP * ldt + DK * lds0 + (out ? CP * ldz + CP * ldw : 0) +
         (out && DK <= 64 ? CP * (DV + 8) : 0);
}
__host__ __device__ constexpr int walk8_lds_bytes(int DK, int DV, bool out) {
  return walk8_lds_elems(DK, DV, out) * 2 + 2 * DK * 4 + (2 * 64 + 4) * 4 + 2 * 64 * 4;
}
constexpr int walk8_groups_per_cu() { return 1; }

// dtype: 0 = f32, 1 = bf16.  Returns hipErrorInvalidValue when no kernel exists
// for (dtype, DK, DV, CP).
hipError_t launch_walk(int dtype, int DK, int DV, int CP, bool output_mode, dim3 grid,
                       const WalkArgs &a, hipStream_t s);
hipError_t launch_walk_f32(int DK, int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                           hipStream_t s);
hipError_t launch_walk8_dk64(int DV, bool output_mode, bool decay, bool den, dim3 grid, const WalkArgs &a,
                             hipStream_t s);
// The lead launch of the bf16 forward: workgroups 0 .. nbh-1 walk segment 0 in output mode and
// write the state after it as the prefix of segment 1; the rest summarise segments 1 .. nsum-1.
hipError_t launch_walk_lead(int DK, int DV, dim3 grid, const WalkArgs &a, hipStream_t s);
hipError_t launch_walk8_lead_dk64(int DV, bool decay, bool den, dim3 grid, const WalkArgs &a, hipStream_t s);
hipError_t launch_walk8_lead_dk128(int DV, bool decay, bool den, dim3 grid, const WalkArgs &a, hipStream_t s);
hipError_t launch_walk8_dk128(int DV, bool output_mode, bool decay, bool den, dim3 grid, const WalkArgs &a,
                              hipStream_t s);
hipError_t launch_scan(int dtype, int DK, int DV, int BH, const ScanArgs &a, hipStream_t s);

// Final state of a forward pass: fold every segment summary, then the tokens after the
// last full chunk, into S, C, U, m, u and write the decode-layout block S | C | m | G | h.
struct StateArgs {
  const float *sums;       // [BH, nseg] summary blocks (padded DK, DV)
  const float *prefix;     // [BH, nseg] exclusive prefix blocks (null when nseg == 1)
  const void *q, *k, *v;   // [BH, n, d|dv], for the tail tokens
  float *state_out;        // [BH, d*d + 2*d*dv + 2*d]
  int n, d, dv, nseg, cps, kc;  // kc: tokens per chunk of the walker
  float log2g;
  int decay_on;
};
hipError_t launch_state(int dtype, int DK, int DV, int BH, const StateArgs &a, hipStream_t s);

struct DecodeArgs {
  float *state;
  const void *q, *k, *v;
  void *out;
  int NH, d, dv;
  float gamma;
  int normalize;
};
hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s);


// Arguments of the backward kernels (hla2_bwd.h, hla2_bwd.hip).
struct BwdArgs {
  const void *q, *k, *v;   // [BH, n, d], [BH, n, d], [BH, n, dv]
  const void *g;           // upstream gradient rows: dout [BH, n, dv], or [BH, n, gld] prepared for the ratio
  void *dq_out, *dk_out, *dv_out;  // [BH, n, d], [BH, n, d], [BH, n, dv]
  const float *prefix;     // forward prefix blocks [BH, nseg] (null when nseg == 1)
  const float *fsum;       // forward summary blocks [BH, nseg-1] (C and m of each segment)
  void *cstate;            // chunk states [BH, nbc] blocks of S0 | U0' (element type)
  float *rsum;             // adjoint summaries [BH, nseg] blocks of Ubar | Shat (fp32)
  float *suffix;           // adjoint states at segment ends [BH, nseg] blocks of Ubar | Shat
  int n, d, dv, gld;       // gld: columns of a row of g
  int nseg, cps, kc;       // segments of cps chunks of kc tokens (the forward's plan)
  int nbc;                 // backward chunks per head
  int nbh;                 // B * H
  float log2g;             // log2(decay)
  int half0 = 0;           // > 0 (two segments): segment 0's forward-state walk in two halves, the
                           // second from fsum block 0 (the first half's summary); chunks of kc tokens
};
// Arguments of the ratio's upstream-gradient preparation.
struct BwdPrepArgs {
  const void *dout, *out;  // [rows, dv]
  const float *den;        // [rows]
  void *gprep;             // [rows, DVP]
  long rows;
  int dv;
};
// BWD_PRE: the forward-state walk and the adjoint summaries, one launch
enum { BWD_PREP = 0, BWD_PRE = 1, BWD_RSCAN = 3, BWD_WALK = 4 };
// Chunk tokens and padded value width of the LDS-operand walkers (backward, AHLA, third order):
// 32-token chunks for fp32 and at d = 128 (LDS), else 64; under the ratio the values gain the
// denominator's ones column, padded to a whole k-tile (16 for fp32, 32 for bf16).
__host__ __device__ constexpr int lds_walk_chunk(bool f32, int DK) { return (f32 || DK == 128) ? 32 : 64; }
__host__ __device__ constexpr int lds_walk_dvp(bool f32, int DV, bool norm) {
  return DV + (norm ? (f32 ? 16 : 32) : 0);
}
// Chunk of the backward walkers: that of lds_walk_chunk, and 32 tokens when the padded value width
// passes 128 (the ratio at dv = 128), where 64-token chunks spill registers.  The host sizes the
// per-chunk state buffer with the same function.
__host__ __device__ constexpr int lds_bwd_chunk(bool f32, int DK, int DVP) {
  return DVP > 128 ? 32 : lds_walk_chunk(f32, DK);
}
// one phase of the backward pass; gL = decay^(tokens per full segment) (reverse scan)
hipError_t launch_bwd(int dtype, int DK, int DV, bool norm, int phase, int BH, const BwdArgs &a,
                      const BwdPrepArgs &pa, float gL, hipStream_t s);


// Arguments of the AHLA kernels (hla2_ahla.hip).
struct AhlaArgs {
  const void *q, *k, *v;   // [BH, n, d], [BH, n, d], [BH, n, dv]
  void *out;               // [BH, n, dv]
  float *den_out;          // [BH, n] or null
  float *prefix;           // [BH, nseg] blocks of P' | E' (DK x DVP each, fp32)
  float *sums;             // [BH, nseg-1] blocks of P' | E' | M (M: DK x DK)
  int n, d, dv;
  int nseg, cps, kc;       // segments of cps chunks of kc tokens
  float log2g;             // log2(decay)
  int normalize;
  int cps0 = 0;            // chunks of segment 0 (0: cps)
  int seg_lo = 0;          // output launch: walks segments seg_lo .. nseg-1
  int nbh = 0;             // heads B*H (lead launch: its first nbh workgroups walk segment 0)
  int first = 0;           // scan: 1 when the prefix of segment 1 is given (lead plans)
  int pfold = 0;           // output launch of a three-segment lead plan without a scan launch: segment 2
                           // folds segment 1's summary onto segment 1's prefix itself
  float gseg = 1.f;        // decay^(tokens per full segment), for pfold
};
// Segment geometry of the AHLA / third-order plans, in chunks of kc tokens.
__host__ __device__ inline int ahla_seg_chunk0(const AhlaArgs &a, int s) {
  return s == 0 ? 0 : (a.cps0 > 0 ? a.cps0 : a.cps) + (s - 1) * a.cps;
}
__host__ __device__ inline int ahla_seg_chunks(const AhlaArgs &a, int s) {
  return s == 0 && a.cps0 > 0 ? a.cps0 : a.cps;
}
// AHLA_LEAD: workgroups 0 .. nbh-1 walk segment 0 in output mode and leave the prefix of
// segment 1; the rest summarise segments 1 .. nseg-2.  AHLA_OUTPUT walks segments
// seg_lo .. nseg-1.
enum { AHLA_SUMMARY = 0, AHLA_SCAN = 1, AHLA_OUTPUT = 2, AHLA_LEAD = 3 };
// one phase of the AHLA forward; gseg = decay^(tokens per full segment) (scan)
hipError_t launch_ahla(int dtype, int DK, int DV, bool norm, int phase, int BH, const AhlaArgs &a, float gseg,
                       hipStream_t s);
// The register-resident walker (hla2_ahla8.hip): bf16, DK = 64, DV = 128, no den; the walk
// phases (AHLA_SUMMARY, AHLA_OUTPUT, AHLA_LEAD) of launch_ahla for that case.
hipError_t launch_ahla8(int phase, int BH, const AhlaArgs &a, hipStream_t s);


// The third-order kernels (hla2_ho3.hip) take the same argument block; their
// prefix blocks are S | P' | W' and their summary blocks S | P' | W' | Q2 | X1 | X2.
using Ho3Args = AhlaArgs;
enum { HO3_SUMMARY = 0, HO3_SCAN = 1, HO3_OUTPUT = 2, HO3_LEAD = 3 };
hipError_t launch_ho3(int dtype, int DK, int DV, bool norm, int phase, int BH, const Ho3Args &a, float gseg,
                      hipStream_t s);
// The register-resident walker (hla2_ho38.hip): bf16, DK = 64, DV = 128, no den; the walk phases
// (HO3_SUMMARY, HO3_OUTPUT, HO3_LEAD) of launch_ho3 for that case.
hipError_t launch_ho38(int phase, int BH, const Ho3Args &a, hipStream_t s);

// The forward pass behind every forward entry point (hla2_api.cpp).  forward_check validates a
// call on the host (everything but the workspace) and reports the workspace bytes it needs;
// forward_run validates again and enqueues the kernels.  dtype is an hla2_dtype_t value.
int forward_check(const void *q, const void *k, const void *v, const void *out, int B, int H, int n, int d, int dv,
                  float decay, int normalize, int chunk, int dtype, const float *den_out, const float *state_out,
                  int segments, size_t *need_out);
int forward_run(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d, int dv,
                float decay, int normalize, int chunk, int dtype, float *den_out, float *state_out,
                void *workspace, size_t workspace_bytes_given, int segments, hipEvent_t const *events,
                hipStream_t stream);

}  // namespace hla2
