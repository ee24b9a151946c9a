// fp32 instantiations of the chunk walker (d, dv <= 64).
#include "hla2_walk.h"

namespace hla2 {

hipError_t launch_walk_f32(int DK, int DV, int CP, bool output_mode, dim3 grid, const WalkArgs &a,
                           hipStream_t s) {
  if (DK != DV) return hipErrorInvalidValue;
  if (DK == 16) {
    if (CP == 16) return launch_walk_t<float, 16, 16, 16>(output_mode, grid, a, s);
    if (CP == 64) return launch_walk_t<float, 16, 16, 64>(output_mode, grid, a, s);
    if (CP == 128) return launch_walk_t<float, 16, 16, 128>(output_mode, grid, a, s);
  } else if (DK == 64) {
    if (CP == 16) return launch_walk_t<float, 64, 64, 16>(output_mode, grid, a, s);
    if (CP == 64) return launch_walk_t<float, 64, 64, 64>(output_mode, grid, a, s);
    if (CP == 128) return launch_walk_t<float, 64, 64, 128>(output_mode, grid, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hla2
