// bf16 instantiations of the chunk walker with d padded to 128.
#include "hla2_walk.h"

namespace hla2 {

hipError_t launch_walk_bf16_dk128(int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                                  hipStream_t s) {
  if (DV == 64 && CP == 64) return launch_walk_t<bf16, 128, 64, 64>(output_mode, grid, a, s);
  if (DV == 64 && CP == 128) return launch_walk_t<bf16, 128, 64, 128>(output_mode, grid, a, s);
  if (DV == 128 && CP == 64) return launch_walk_t<bf16, 128, 128, 64>(output_mode, grid, a, s);
  if (DV == 128 && CP == 128) return launch_walk_t<bf16, 128, 128, 128>(output_mode, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
