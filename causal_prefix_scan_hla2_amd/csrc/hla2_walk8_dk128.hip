// bf16 chunk-walker instantiations with d padded to 128 (the 8-wave walker of hla2_walk8.h).
#include "hla2_walk8.h"

namespace hla2 {

hipError_t launch_walk8_dk128(int DV, bool output_mode, bool decay, bool den, dim3 grid, const WalkArgs &a,
                             hipStream_t s) {
  if (DV == 64) return launch_walk8_t<128, 64>(output_mode, decay, den, grid, a, s);
  if (DV == 128) return launch_walk8_t<128, 128>(output_mode, decay, den, grid, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_walk8_lead_dk128(int DV, bool decay, bool den, dim3 grid, const WalkArgs &a, hipStream_t s) {
  if (DV == 64) return launch_walk8_lead_t<128, 64>(decay, den, grid, a, s);
  if (DV == 128) return launch_walk8_lead_t<128, 128>(decay, den, grid, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hla2
