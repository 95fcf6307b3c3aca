// decode_d128.hip -- instantiations of the fused decode kernel for d = 128.
#include "decode_kernel.h"

namespace la {
template hipError_t launch_decode_dim<128>(const DecodeArgs &, int, bool, hipStream_t);
}  // namespace la
