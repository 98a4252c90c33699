// Chunked prefill (MFMA) -- placeholder until the kernel lands.
#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fe
