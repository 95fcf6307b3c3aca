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
// Only the history hand-off of shortconv_prefill (the fused prefill computes
// the outputs itself).
hipError_t launch_shortconv_handoff(const ConvPrefillArgs &a, hipStream_t stream);

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
    // fused short conv: x holds the pre-conv q|k|v projections [T, C] and the
    // conv + SiLU runs inside the prefill's loads (q, k, v unused)
    bool conv;
    const void *x;
    int C;
    const float *w, *bias;
    const void *conv_pool;
    int64_t conv_stride;
    int conv_dtype;
};
size_t prefill_ws_bytes(int N, int T, int Hqk, int Hv, int D, int mode);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);


// ---- speculative decode: verify, exact commit, conv-window scatter, state
//      tracking copy ----
struct RingArgs {
    int L;                          // ring depth, a power of two
    void *d, *k, *rawv, *rawk;      // [num_rows, Hv, L, 128] io dtype
    float *g, *beta;                // [num_rows, Hv, L, 128 (KDA) or 1], [num_rows, Hv, L]
};

struct VerifyArgs {
    int B, D, Hqk, Hv, G, C;        // D = draft tokens per request (max)
    const int32_t *n_tok;           // [B] tokens used per request
    const void *x;                  // [B, D, C] io dtype
    int io_dtype;
    const float *w, *bias;          // conv weights or nullptr (x is post-conv)
    const void *conv_pool;
    int64_t conv_stride;
    int conv_dtype;
    const float *g, *beta;          // [B, D, Hv, 128] / [B, D, Hv]; [B, D, Hv]
    const int32_t *slots;
    int num_rows;
    const void *ssm_pool;
    int64_t ssm_stride;
    void *out;                      // [B, D, Hv, 128] io dtype
    void *windows;                  // [B, D, 3, C] conv dtype
    RingArgs ring;
    const int32_t *ring_base;       // [B]
    float eps, scale;
};
hipError_t launch_verify(const VerifyArgs &a, int state_dtype, bool kda, hipStream_t stream);

struct CommitArgs {
    int B, Hv;
    const int32_t *accepted, *slots;
    int num_rows;
    void *ssm_pool;
    int64_t ssm_stride;
    int io_dtype;                   // dtype of the ring's vectors
    RingArgs ring;
    const int32_t *ring_base;
    float eps;
};
hipError_t launch_commit(const CommitArgs &a, int state_dtype, bool kda, hipStream_t stream);

struct ScatterArgs {
    int B, D, C;
    const uint8_t *mask;            // [B] or nullptr
    const int32_t *slots, *step;    // [B]
    const void *windows;            // [B, D, 3, C] conv dtype
    void *conv_pool;
    int64_t conv_stride;
    int conv_dtype;
    int num_rows;
};
hipError_t launch_conv_scatter(const ScatterArgs &a, hipStream_t stream);

struct TrackArgs {
    int B;
    const uint8_t *mask;            // [B] or nullptr
    const int32_t *src, *dst;       // [B]
    char *conv_pool, *ssm_pool;     // byte views
    int64_t conv_stride_b, conv_row_b, ssm_stride_b, ssm_row_b;  // bytes
    int num_rows;
};
hipError_t launch_track_copy(const TrackArgs &a, hipStream_t stream);


struct FoldArgs {
    int B, Hv;
    const int32_t *m, *slots, *dst;  // [B]; dst == nullptr: in place
    int num_rows;
    void *ssm_pool;
    int64_t ssm_stride;
    int io_dtype;                    // dtype of the ring's vectors, q and out
    RingArgs ring;
    const int32_t *ring_base;
    const void *q;                   // [B, Hv, 128] raw queries or nullptr
    void *out;                       // [B, Hv, 128] or nullptr
    float eps, scale;
};
hipError_t launch_fold(const FoldArgs &a, int state_dtype, bool kda, hipStream_t stream);

}  // namespace la
