// la_internal.h -- argument bundles and kernel launchers behind the C ABI.
// The host entry points in la_api.cpp validate arguments and call these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

struct DecodeArgs {
    int B, Hqk, Hv, G, C;           // G = Hv / Hqk value heads per q/k head
    const void *x;                  // [B, C] io dtype
    int io_dtype;
    const float *w, *bias;          // [C, 4], [C] or nullptr
    void *conv_pool;                // rows [3, C]
    int64_t conv_stride;            // elements between pool rows
    int conv_dtype;
    const float *g, *beta;          // KDA [B, Hv, D] / GDN [B, Hv]; [B, Hv]
    const int32_t *slots;           // [B]
    int num_rows;
    void *ssm_pool;                 // rows [Hv, D, D]
    int64_t ssm_stride;             // elements between pool rows
    void *out;                      // [B, Hv, D] io dtype
    float eps, scale;
};

// Fused decode step (conv + SiLU + L2 norm + gated delta rule).
hipError_t launch_decode(const DecodeArgs &a, int D, int state_dtype, bool kda,
                         hipStream_t stream);

struct ConvStepArgs {
    int B, C;
    const void *x;
    int x_dtype;
    const float *w, *bias;
    void *conv_pool;
    int64_t conv_stride;
    int conv_dtype;
    int num_rows;
    const int32_t *slots;
    void *y;
};
hipError_t launch_shortconv_update(const ConvStepArgs &a, hipStream_t stream);

struct ConvPrefillArgs {
    int N, T, C;
    const void *x;
    int io_dtype;
    const int32_t *cu, *slot_in, *slot_out;
    const float *w, *bias;
    void *conv_pool;
    int64_t conv_stride;
    int conv_dtype;
    int num_rows;
    void *y;
};
hipError_t launch_shortconv_prefill(const ConvPrefillArgs &a, hipStream_t stream);

struct PrefillArgs {
    int N, T, Hqk, Hv, G, D;
    const void *q, *k, *v;
    int64_t q_stride, k_stride, v_stride;
    int io_dtype;
    const float *g, *beta;
    const int32_t *cu, *slot_in, *slot_out;
    int num_rows;
    void *ssm_pool;
    int64_t ssm_stride;
    int state_dtype;
    void *out;
    float eps, scale;
    int mode;
    bool kda;
    void *ws;
    size_t ws_bytes;
};
size_t prefill_ws_bytes(int N, int T, int Hqk, int Hv, int D, int mode);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

}  // namespace la
