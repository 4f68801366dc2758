// Chunked prefill: not built yet; the C ABI reports PA_ERR_UNSUPPORTED.
#include "pa_launch.h"

namespace pkv {
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pkv
