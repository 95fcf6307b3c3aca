// shortconv.hip -- the kernel-size-4 depthwise causal short conv + SiLU.
//
// The conv runs over the projected q|k|v channels; each channel mixes the
// current token with the three before it, kept per slot as a 3-row history
// (xxmr.cn/news/181459, "Conv state" passage; hotelren.com/news/5417338
// section 2.1).  Tap 3 multiplies the current token and history row 0 is the
// oldest token:  y = SiLU(w0 h0 + w1 h1 + w2 h2 + w3 x + bias).
//
// All kernels are streaming passes with the channel index contiguous across
// lanes, so every access is coalesced.  The prefill output kernel moves
// 16 bytes of channels per lane and slides the 4-token window along a run of
// tokens, so each input row is read once (plus three rows at a run's start);
// the hand-off kernel writes each sequence's first three outputs.
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

// Outputs, scalar path (any C).  grid (ceil(C / 256), ceil(T / kTokPerBlock)),
// block 256.  The pool is only read here (as in the vector path); the history
// is written by the next kernel, so a sequence whose slot_in equals its
// slot_out reads its old history safely.
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

// Vector path (C a multiple of 8): lane = 16 bytes of channels, thread = a
// run of kConvTok tokens.  grid (ceil(C / (256 V)), ceil(T / kConvTok)),
// block 256.  Only tokens whose whole window lies inside their own sequence
// (t - 3 >= the sequence's first token) are computed here, from input rows
// loaded up front; the first three tokens of every sequence need the slot
// history and are written by the hand-off kernel.  No load is issued inside
// the token loop, so stores never wait on loads.  Same arithmetic, in the
// same order, as the scalar kernel.
constexpr int kConvTok = 16;
template <typename IOT>
__global__ void __launch_bounds__(256) shortconv_prefill_vec_kernel(ConvPrefillArgs a)
{
    constexpr int V = Stor<IOT>::kPer16B;  // channels per lane
    const int c0 = (blockIdx.x * 256 + threadIdx.x) * V;
    if (c0 >= a.C) return;
    const int t0 = blockIdx.y * kConvTok;
    const int nt = min(kConvTok, a.T - t0);
    const IOT *x = static_cast<const IOT *>(a.x);
    IOT *y = static_cast<IOT *>(a.y);

    // The run's first sequence and its bounds, and the weights, before the
    // row loads (so waiting for them does not wait for the rows).  A missing
    // bias reads the weights instead and is scaled by 0: no branch around a load.
    int n = find_seq(a.cu, a.N, t0);
    int s0 = a.cu[n], e0 = a.cu[n + 1];
    bool ok0 = seq_slots_ok(a, n);
    const float bias_on = a.bias ? 1.f : 0.f;
    const float *bsrc = a.bias ? a.bias : a.w;
    float4 wc[V];
    float bs[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        wc[e] = reinterpret_cast<const float4 *>(a.w)[c0 + e];
        bs[e] = bsrc[c0 + e];
    }
    // rows t0 - 3 .. t0 + kConvTok - 1 (clamped into [0, T)), issued back to back
    uint4 raw[kConvTok + 3];
#pragma unroll
    for (int i = 0; i < kConvTok + 3; ++i) {
        const int t = min(max(t0 - 3 + i, 0), a.T - 1);
        raw[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)t * a.C + c0);
    }
    // Token masks of the run: bit i set in `comp` = compute token t0 + i here
    // (its window lies inside its sequence), in `zero` = its sequence is
    // skipped (out-of-range slot), so its output is zero.
    uint32_t comp = 0, zero = 0;
    const int tend = t0 + nt;
    auto mark = [&](int st, int en, bool ok) {
        const int lo = max(st + (ok ? 3 : 0), t0), hi = min(en, tend);
        if (lo < hi) {
            const uint32_t bits = ((1u << (hi - lo)) - 1u) << (lo - t0);
            if (ok) comp |= bits;
            else zero |= bits;
        }
    };
    mark(s0, e0, ok0);
    while (e0 < tend) {  // further sequences starting inside the run (rare)
        ++n;
        s0 = a.cu[n];
        e0 = a.cu[n + 1];
        mark(s0, e0, seq_slots_ok(a, n));
    }
    float win[4][V];
#pragma unroll
    for (int r = 0; r < 3; ++r) Stor<IOT>::unpack(raw[r], win[r + 1]);
#pragma unroll
    for (int i = 0; i < kConvTok; ++i) {
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int e = 0; e < V; ++e) win[r][e] = win[r + 1][e];
        Stor<IOT>::unpack(raw[i + 3], win[3]);
        // computed unconditionally (branch-free); the masks only gate the store
        const bool c = (comp >> i) & 1u;
        float yv[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float v = conv4(wc[e], bs[e] * bias_on, win[0][e], win[1][e], win[2][e], win[3][e]);
            yv[e] = c ? v : 0.f;
        }
        if (c || ((zero >> i) & 1u))
            *reinterpret_cast<uint4 *>(y + (int64_t)(t0 + i) * a.C + c0) = Stor<IOT>::pack(yv);
    }
}

// History hand-off.  grid (ceil(C / 256), N), block 256.  The last three
// pre-conv inputs of sequence n (older history shifted in for sequences
// shorter than three tokens) go to row slot_out[n]; each lane reads all it
// needs before writing, so slot_in == slot_out is safe.  With `head_outputs`
// (the vector path) it also writes the outputs of the sequence's first
// min(3, len) tokens, whose windows reach into the slot_in history.
__global__ void __launch_bounds__(256) shortconv_prefill_state_kernel(ConvPrefillArgs a,
                                                                      int head_outputs)
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
    if (head_outputs) {
        const float4 wc = reinterpret_cast<const float4 *>(a.w)[c];
        const float bias = a.bias ? a.bias[c] : 0.f;
        float xin[3];
#pragma unroll
        for (int j = 0; j < 3; ++j)
            xin[j] = j < len ? load_elem(a.x, (int64_t)(start + j) * a.C + c, a.io_dtype) : 0.f;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (j >= len) break;
            float win[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pos = j - 3 + r;  // position relative to the sequence start
                win[r] = pos >= 0 ? xin[pos] : h[pos + 3];
            }
            store_elem(a.y, (int64_t)(start + j) * a.C + c, a.io_dtype,
                       conv4(wc, bias, win[0], win[1], win[2], win[3]));
        }
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
    const bool vec = a.C % 8 == 0;
    if (a.T > 0 && vec) {
        const int V = a.io_dtype ? 8 : 4;
        dim3 g1((unsigned)((a.C / V + 255) / 256), (unsigned)((a.T + kConvTok - 1) / kConvTok));
        if (a.io_dtype)
            hipLaunchKernelGGL(shortconv_prefill_vec_kernel<bf16_t>, g1, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(shortconv_prefill_vec_kernel<float>, g1, dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (a.T > 0) {
        dim3 g1(cb, (unsigned)((a.T + kTokPerBlock - 1) / kTokPerBlock));
        hipLaunchKernelGGL(shortconv_prefill_out_kernel, g1, dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 g2(cb, (unsigned)a.N);
    hipLaunchKernelGGL(shortconv_prefill_state_kernel, g2, dim3(256), 0, stream, a, (int)vec);
    return hipGetLastError();
}

hipError_t launch_shortconv_handoff(const ConvPrefillArgs &a, hipStream_t stream)
{
    dim3 g2((unsigned)((a.C + 255) / 256), (unsigned)a.N);
    hipLaunchKernelGGL(shortconv_prefill_state_kernel, g2, dim3(256), 0, stream, a, 0);
    return hipGetLastError();
}

}  // namespace la
