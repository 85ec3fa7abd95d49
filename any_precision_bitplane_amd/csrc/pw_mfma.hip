// Dequant-to-LDS MFMA kernels for experts with many tokens (prefill).
#include "pw_device.h"
#include "pw_internal.h"

namespace pw {

hipError_t launch_mfma_gate_up(const ExpertArgs&, const uint16_t*, uint16_t*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_mfma_down(const ExpertArgs&, const uint16_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pw
