// decode_d64.hip -- instantiations of the fused decode kernel for d = 64.
#include "decode_kernel.h"

namespace la {
template hipError_t launch_decode_dim<64>(const DecodeArgs &, int, bool, hipStream_t);
}  // namespace la
