// probe.hip -- test support only: evaluates the library's device math helpers
// (la_device.h: exp_acc, fast_exp, silu) element-wise on the GPU, so
// tests/test_gpu_device_math.py can bound their error against fp64 libm.
// Not part of libla.
#include <hip/hip_runtime.h>

#include "la_device.h"

namespace {

__global__ void eval_kernel(const float *x, float *y, int n, int which)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float v = x[i];
    y[i] = which == 0 ? la::exp_acc(v) : which == 1 ? la::fast_exp(v) : la::silu(v);
}

}  // namespace

// x, y: device buffers of n floats.  which: 0 exp_acc, 1 fast_exp, 2 silu.
// Returns 0, or the HIP error code of the launch or of the synchronisation.
extern "C" int devmath_eval(const float *x, float *y, int n, int which)
{
    if (n <= 0) return 0;
    hipLaunchKernelGGL(eval_kernel, dim3((n + 255) / 256), dim3(256), 0, nullptr, x, y, n, which);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return (int)e;
}
