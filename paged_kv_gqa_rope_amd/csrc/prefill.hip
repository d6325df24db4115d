// Context-phase MFMA kernel (placeholder launcher until it lands).
#include "kernels.h"

namespace pkv {
hipError_t launch_prefill(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pkv
