// shortconv.hip -- the kernel-size-4 depthwise causal short conv + SiLU.
//
// The conv runs over the projected q|k|v channels; each channel mixes the
// current token with the three before it, kept per slot as a 3-row history
// (xxmr.cn/news/181459, "Conv state" passage; hotelren.com/news/5417338
// section 2.1).  Tap 3 multiplies the current token and history row 0 is the
// oldest token:  y = SiLU(w0 h0 + w1 h1 + w2 h2 + w3 x + bias).
//
// Both kernels are streaming elementwise passes: one lane per channel, the
// channel index contiguous across lanes so every access is coalesced.
#include "la_device.h"
#include "la_internal.h"

namespace la {

__device__ __forceinline__ float conv4(const float4 wc, float bias, float h0, float h1,
                                       float h2, float x)
{
    float acc = bias;
    acc = fmaf(wc.x, h0, acc);
    acc = fmaf(wc.y, h1, acc);
    acc = fmaf(wc.z, h2, acc);
    acc = fmaf(wc.w, x, acc);
    return silu(acc);
}

// ---- decode: one token per batch entry, history rolled in place -----------
// grid (ceil(C / 256), B), block 256.
__global__ void __launch_bounds__(256) shortconv_update_kernel(ConvStepArgs a)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int b = blockIdx.y;
    if (c >= a.C) return;
    const int slot = a.slots[b];
    const int64_t xi = (int64_t)b * a.C + c;
    if (slot < 0 || slot >= a.num_rows) {  // skipped entry
        store_elem(a.y, xi, a.x_dtype, 0.f);
        return;
    }
    const int csz = a.conv_dtype ? 2 : 4;
    char *cs = static_cast<char *>(a.conv_pool) + (int64_t)slot * a.conv_stride * csz;
    const float xv = load_elem(a.x, xi, a.x_dtype);
    const float h0 = load_elem(cs, c, a.conv_dtype);
    const float h1 = load_elem(cs, a.C + c, a.conv_dtype);
    const float h2 = load_elem(cs, 2 * a.C + c, a.conv_dtype);
    const float4 wc = reinterpret_cast<const float4 *>(a.w)[c];
    const float y = conv4(wc, a.bias ? a.bias[c] : 0.f, h0, h1, h2, xv);
    store_elem(a.y, xi, a.x_dtype, y);
    store_elem(cs, c, a.conv_dtype, h1);  // exact round trips: bit copies
    store_elem(cs, a.C + c, a.conv_dtype, h2);
    store_elem(cs, 2 * a.C + c, a.conv_dtype, xv);
}

hipError_t launch_shortconv_update(const ConvStepArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)((a.C + 255) / 256), (unsigned)a.B);
    hipLaunchKernelGGL(shortconv_update_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---- prefill over packed sequences ----------------------------------------

// Sequence holding token t: the n with cu[n] <= t < cu[n+1].
__device__ __forceinline__ int find_seq(const int32_t *cu, int N, int t)
{
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bool seq_slots_ok(const ConvPrefillArgs &a, int n)
{
    const int si = a.slot_in[n], so = a.slot_out[n];
    return si < a.num_rows && so >= 0 && so < a.num_rows;
}

// Outputs.  grid (ceil(C / 256), ceil(T / kTokPerBlock)), block 256.  The
// pool is only read here; the history is written by the next kernel, so a
// sequence whose slot_in equals its slot_out reads its old history safely.
constexpr int kTokPerBlock = 8;
__global__ void __launch_bounds__(256) shortconv_prefill_out_kernel(ConvPrefillArgs a)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= a.C) return;
    const float4 wc = reinterpret_cast<const float4 *>(a.w)[c];
    const float bias = a.bias ? a.bias[c] : 0.f;
    const int csz = a.conv_dtype ? 2 : 4;
    const int t0 = blockIdx.y * kTokPerBlock;
    const int t1 = min(a.T, t0 + kTokPerBlock);
    for (int t = t0; t < t1; ++t) {
        const int n = find_seq(a.cu, a.N, t);
        const int start = a.cu[n];
        const int64_t yi = (int64_t)t * a.C + c;
        if (!seq_slots_ok(a, n)) {
            store_elem(a.y, yi, a.io_dtype, 0.f);
            continue;
        }
        const int si = a.slot_in[n];
        const char *cs = si >= 0 ? static_cast<const char *>(a.conv_pool) +
                                       (int64_t)si * a.conv_stride * csz
                                 : nullptr;
        float win[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = t - 3 + i;
            if (pos >= start) win[i] = load_elem(a.x, (int64_t)pos * a.C + c, a.io_dtype);
            else win[i] = cs ? load_elem(cs, (int64_t)(pos - start + 3) * a.C + c, a.conv_dtype)
                             : 0.f;
        }
        store_elem(a.y, yi, a.io_dtype, conv4(wc, bias, win[0], win[1], win[2], win[3]));
    }
}

// History hand-off.  grid (ceil(C / 256), N), block 256.  The last three
// pre-conv inputs of sequence n (older history shifted in for sequences
// shorter than three tokens) go to row slot_out[n]; each lane reads all it
// needs before writing, so slot_in == slot_out is safe.
__global__ void __launch_bounds__(256) shortconv_prefill_state_kernel(ConvPrefillArgs a)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int n = blockIdx.y;
    if (c >= a.C || !seq_slots_ok(a, n)) return;
    const int csz = a.conv_dtype ? 2 : 4;
    const int start = a.cu[n], len = a.cu[n + 1] - start;
    const int si = a.slot_in[n];
    float h[3] = {0.f, 0.f, 0.f};
    if (si >= 0) {
        const char *cs = static_cast<const char *>(a.conv_pool) + (int64_t)si * a.conv_stride * csz;
#pragma unroll
        for (int r = 0; r < 3; ++r) h[r] = load_elem(cs, (int64_t)r * a.C + c, a.conv_dtype);
    }
    float nh[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const int pos = len - 3 + r;
        nh[r] = pos >= 0 ? load_elem(a.x, (int64_t)(start + pos) * a.C + c, a.io_dtype)
                         : h[pos + 3];
    }
    char *out = static_cast<char *>(a.conv_pool) + (int64_t)a.slot_out[n] * a.conv_stride * csz;
#pragma unroll
    for (int r = 0; r < 3; ++r) store_elem(out, (int64_t)r * a.C + c, a.conv_dtype, nh[r]);
}

hipError_t launch_shortconv_prefill(const ConvPrefillArgs &a, hipStream_t stream)
{
    const unsigned cb = (unsigned)((a.C + 255) / 256);
    if (a.T > 0) {
        dim3 g1(cb, (unsigned)((a.T + kTokPerBlock - 1) / kTokPerBlock));
        hipLaunchKernelGGL(shortconv_prefill_out_kernel, g1, dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 g2(cb, (unsigned)a.N);
    hipLaunchKernelGGL(shortconv_prefill_state_kernel, g2, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace la
