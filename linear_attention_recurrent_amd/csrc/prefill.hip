// prefill.hip -- chunked prefill (placeholder until the kernels land).
#include "la_device.h"
#include "la_internal.h"

namespace la {

size_t prefill_ws_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace la
