// decode_d16.hip -- instantiations of the fused decode kernel for d = 16.
#include "decode_kernel.h"

namespace la {
template hipError_t launch_decode_dim<16>(const DecodeArgs &, int, bool, hipStream_t);
}  // namespace la
