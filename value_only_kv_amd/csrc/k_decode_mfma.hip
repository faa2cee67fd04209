// k_decode_mfma.hip - matrix-core split decode (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "gva_internal.h"

namespace gva {
hipError_t launch_decode_mfma(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gva
