// bf16 chunk-walker instantiations with d padded to 64 (the 8-wave walker of hla2_walk8.h).
#include "hla2_walk8.h"

namespace hla2 {

hipError_t launch_walk8_dk64(int DV, bool output_mode, bool decay, bool den, dim3 grid, const WalkArgs &a,
                             hipStream_t s) {
  if (DV == 64) return launch_walk8_t<64, 64>(output_mode, decay, den, grid, a, s);
  if (DV == 128) return launch_walk8_t<64, 128>(output_mode, decay, den, grid, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_walk8_lead_dk64(int DV, bool decay, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
  if (DV == 64) return launch_walk8_lead_t<64, 64>(decay, den, grid, a, s);
  if (DV == 128) return launch_walk8_lead_t<64, 128>(decay, den, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
