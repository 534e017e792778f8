// STA backward, bf16 in/out (placeholder until the MFMA kernels land).
#include "kernels.h"

namespace sta {

bool bwd_bf16_supported(int D, int L) {
  (void)D;
  (void)L;
  return false;
}

hipError_t launch_bwd_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                           const uint16_t*, const float*, uint16_t*, uint16_t*, uint16_t*, float*,
                           const Geometry&, const HeadTable&, int, int, int, float, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace sta
