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
};

// Arguments of the segment-level exclusive scan.
struct ScanArgs {
  const float *sums;  // [BH, nseg-1] summary blocks
  float *prefix;      // [BH, nseg] prefix blocks
  int nseg;
  float gamma_seg;    // decay^(tokens per full segment)
};

// Per-(b,h,segment) block sizes in floats, for padded dims DK, DV.
//   summary block: S[DK*DK] | C[DK*DV] | U[DK*DV] | m[DK] | u[DK]
//   prefix block:  S0[DK*DK] | U0[DK*DV] | u0[DK]
__host__ __device__ inline long sum_block_floats(int DK, int DV) { return (long)DK * DK + 2L * DK * DV + 2L * DK; }
__host__ __device__ inline long prefix_block_floats(int DK, int DV) { return (long)DK * DK + (long)DK * DV + DK; }

// dtype: 0 = f32, 1 = bf16.  Returns hipErrorInvalidValue when no kernel exists
// for (dtype, DK, DV, CP).
hipError_t launch_walk(int dtype, int DK, int DV, int CP, bool output_mode, dim3 grid,
                       const WalkArgs &a, hipStream_t s);
hipError_t launch_walk_f32(int DK, int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                           hipStream_t s);
hipError_t launch_walk_bf16_dk64(int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                                 hipStream_t s);
hipError_t launch_walk_bf16_dk128(int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                                  hipStream_t s);
hipError_t launch_scan(int DK, int DV, int BH, const ScanArgs &a, hipStream_t s);

struct DecodeArgs {
  float *state;
  const void *q, *k, *v;
  void *out;
  int NH, d, dv;
  float gamma;
  int normalize;
};
hipError_t launch_decode(int dtype, const DecodeArgs &a, hipStream_t s);

}  // namespace hla2
