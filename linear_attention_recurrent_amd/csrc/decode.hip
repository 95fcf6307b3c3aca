// decode.hip -- dispatch of the fused KDA / GDN decode step by head dim.  The
// kernel itself is in decode_kernel.h; each head dim is instantiated in its
// own translation unit (decode_d*.hip) so they compile in parallel.
#include "decode_kernel.h"

namespace la {

extern template hipError_t launch_decode_dim<16>(const DecodeArgs &, int, bool, hipStream_t);
extern template hipError_t launch_decode_dim<32>(const DecodeArgs &, int, bool, hipStream_t);
extern template hipError_t launch_decode_dim<64>(const DecodeArgs &, int, bool, hipStream_t);
extern template hipError_t launch_decode_dim<128>(const DecodeArgs &, int, bool, hipStream_t);

hipError_t launch_decode(const DecodeArgs &a, int D, int state_dtype, bool kda,
                         hipStream_t stream)
{
    switch (D) {
    case 16: return launch_decode_dim<16>(a, state_dtype, kda, stream);
    case 32: return launch_decode_dim<32>(a, state_dtype, kda, stream);
    case 64: return launch_decode_dim<64>(a, state_dtype, kda, stream);
    case 128: return launch_decode_dim<128>(a, state_dtype, kda, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace la
