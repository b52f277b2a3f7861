// Causal FAVOR+ (placeholder until the chunked scan lands).
#include "favor_device.hpp"
#include "favor_internal.hpp"

namespace favor {
hipError_t launch_causal(const Plan&, const Tensors&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace favor
