// decode_d32.hip -- instantiations of the fused decode kernel for d = 32.
#include "decode_kernel.h"

namespace la {
template hipError_t launch_decode_dim<32>(const DecodeArgs &, int, bool, hipStream_t);
}  // namespace la
