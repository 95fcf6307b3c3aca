// decode_kernel.h -- the fused decode kernel template (instantiated per head
// dim in decode_d*.hip; dispatched from decode.hip).
//
// What it computes (the decode kernel's steps in "SGLang之KV Cache内存池机制",
// section 8.5; the exact replay order in the ReplaySSM passage of
// xxmr.cn/news/181459; the short conv in that page's "Conv state" passage):
//   y   = SiLU(conv4(history, x))          short conv over q|k|v channels
//   q,k = y_q / sqrt(|y_q|^2 + eps), ...   L2 norm
//   S' = S Diag(exp g); u = S' k; d = beta (v - u); S = S' + d k^T
//   o   = scale S q = scale (S' q + d (k . q))
// in place on the slot-indexed pools.
//
// Work decomposition.  One workgroup per (request b, q/k head kh) owns the
// G = H_v / H_qk value heads that share that q/k head, so it is the only
// reader and writer of every conv-state channel it touches.
//
// State streaming.  Row i of a head's state (d_k contiguous) is split over
// LPR lanes holding 16 bytes each (8 bf16 or 4 fp32), so one wave instruction
// moves RPW = 64 / LPR consecutive rows = 1 KB contiguous: fully coalesced.
// Each wave owns a contiguous band of RW rows per head; the row loads and
// stores carry the non-temporal hint.  Both row reductions
// (S'k and S'q) come out of one pass over the registers (DPP adds inside the
// LPR-lane group, bit-identical in every lane), the update is applied in
// registers and the row is stored back: the state crosses HBM once each way.
//
// Latency hiding.  Each wave issues its few prologue loads (x, conv
// history, conv weights, gates) and computes the conv + SiLU prologue: with
// one value head per workgroup the waves split the q and k channels and one
// workgroup barrier publishes the q/k conv outputs (with several heads per
// workgroup every wave convolves all of them itself, and the shared q/k
// history is rolled after a barrier at the end); every wave forms the L2
// norms.  Only then does a wave issue all of its state-row loads; it
// consumes the rows in issue order, storing each as soon as it is updated.
// (Issuing the rows before the prologue, so they are in flight meanwhile,
// was slower: the small prologue loads then wait behind every workgroup's
// rows.)  With G > 1 the next head's loads are issued before the current
// head is computed.
#pragma once

#include "la_device.h"
#include "la_internal.h"

#include <type_traits>

namespace la {

template <int D, typename ST> struct DecodeCfg {
    static constexpr int EPL = Stor<ST>::kPer16B;   // elements per lane per row
    static constexpr int LPR = D / EPL;             // lanes per row
    static constexpr int RPW = 64 / LPR;            // rows per wave instruction
    static constexpr int RI = (D + RPW - 1) / RPW;  // wave instructions per head
    static constexpr int NW_MAX = sizeof(ST) == 4 ? 8 : 4;
    static constexpr int NW = RI < NW_MAX ? RI : NW_MAX;  // waves per workgroup
    static constexpr int NJ = RI / NW;              // row instructions per lane
    static constexpr int NT = 64 * NW;              // threads per workgroup
    static constexpr int RW = D < NJ * RPW ? D : NJ * RPW;  // rows per wave per head
    static constexpr int QKL = (D + 63) / 64;       // q (or k) channels per lane, whole-head prologue
    static constexpr int QS = D / NW;               // q (and k) channels per wave, split prologue
    static constexpr int LDS_SPLIT = 2 * D + NW * RW;   // floats: shared q, k outputs; v bands
    static constexpr int LDS_WHOLE = NW * (2 * D + RW); // floats: per wave q, k, v band
    static_assert(QS * NW == D && QS <= 32, "q/k channels split over the waves, 32 lanes each");
    static_assert(LPR >= 1 && LPR <= 32, "row must fit in half a wave");
    static_assert(RI % NW == 0, "rows must split evenly over waves");
    static_assert(NJ <= LPR, "one output lane per row instruction");
    static_assert(RW <= 64, "one v channel per lane");
};

// One conv tap set: history h0..h2 (oldest first) and the current input,
// held as raw stored bits until used.  All dtypes are template parameters and
// nothing is converted at the load site, so the prologue loads are
// straight-line code issued back to back, ahead of the state rows.
template <typename T> struct RawOf { using type = float; };
template <> struct RawOf<bf16_t> { using type = uint16_t; };

__device__ __forceinline__ float raw_f32(float v) { return v; }
__device__ __forceinline__ float raw_f32(uint16_t v) { return bf16_to_f32(v); }

template <typename IOT, typename CT> struct ConvIn {
    typename RawOf<CT>::type h0, h1, h2;
    typename RawOf<IOT>::type x;
    float4 w;
    float bias;
};

template <typename IOT, typename CT, bool CONV>
__device__ __forceinline__ void load_conv_in(ConvIn<IOT, CT> &ci, const DecodeArgs &a,
                                             const CT *cs, int64_t xrow, int c)
{
    using RI = typename RawOf<IOT>::type;
    using RC = typename RawOf<CT>::type;
    ci.x = static_cast<const RI *>(a.x)[xrow + c];
    if constexpr (CONV) {
        const RC *h = reinterpret_cast<const RC *>(cs);
        ci.h0 = h[c];
        ci.h1 = h[a.C + c];
        ci.h2 = h[2 * a.C + c];
        ci.w = reinterpret_cast<const float4 *>(a.w)[c];
        // A missing bias reads the (always valid) weights instead and is
        // scaled by 0 in conv_out: no branch around the load.
        ci.bias = (a.bias ? a.bias : a.w)[c];
    }
}

template <bool CONV, typename IOT, typename CT>
__device__ __forceinline__ float conv_out(const ConvIn<IOT, CT> &ci, float bias_on)
{
    const float x = raw_f32(ci.x);
    if constexpr (!CONV) return x;
    float acc = ci.bias * bias_on;
    acc = fmaf(ci.w.x, raw_f32(ci.h0), acc);
    acc = fmaf(ci.w.y, raw_f32(ci.h1), acc);
    acc = fmaf(ci.w.z, raw_f32(ci.h2), acc);
    acc = fmaf(ci.w.w, x, acc);
    return silu(acc);
}

// History roll of one channel: rows 1, 2 move to 0, 1 and the input becomes
// row 2 -- raw bit copies (the input is converted only when the I/O and conv
// dtypes differ).
template <typename IOT, typename CT>
__device__ __forceinline__ void roll_history(const ConvIn<IOT, CT> &ci, const DecodeArgs &a,
                                             CT *cs, int c)
{
    using RC = typename RawOf<CT>::type;
    RC *h = reinterpret_cast<RC *>(cs);
    h[c] = ci.h1;
    h[a.C + c] = ci.h2;
    if constexpr (std::is_same<IOT, CT>::value) h[2 * a.C + c] = ci.x;
    else st<CT>(cs, 2 * a.C + c, raw_f32(ci.x));
}

template <int D, typename ST>
__device__ __forceinline__ void load_rows(uint4 *buf, const ST *S, int wave, int lane)
{
    using Cfg = DecodeCfg<D, ST>;
    const int col0 = (lane % Cfg::LPR) * Cfg::EPL;
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j) {
        const int r = (wave * Cfg::NJ + j) * Cfg::RPW + lane / Cfg::LPR;
        if (D >= Cfg::RPW || r < D)
            buf[j] = ld_stream(S + (int64_t)r * D + col0);
        else
            buf[j] = make_uint4(0, 0, 0, 0);
    }
}

// Per-head gate values of this lane's columns.
template <int D, typename ST, bool KDA>
__device__ __forceinline__ void load_gates(float (&gl)[Stor<ST>::kPer16B], float &beta,
                                           const DecodeArgs &a, int b, int h, int col0)
{
    constexpr int EPL = Stor<ST>::kPer16B;
    if constexpr (KDA) {
        const float *gp = a.g + ((int64_t)b * a.Hv + h) * D + col0;
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            const float4 g4 = *reinterpret_cast<const float4 *>(gp + e);
            gl[e] = g4.x; gl[e + 1] = g4.y; gl[e + 2] = g4.z; gl[e + 3] = g4.w;
        }
    } else {
        const float g1 = a.g[(int64_t)b * a.Hv + h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) gl[e] = g1;
    }
    beta = a.beta[(int64_t)b * a.Hv + h];
}

template <int D, typename ST, typename IOT, typename CT, bool KDA, int GT, bool CONV>
__global__ void __launch_bounds__((DecodeCfg<D, ST>::NT)) decode_kernel(DecodeArgs a)
{
    using Cfg = DecodeCfg<D, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ;
    constexpr int RW = Cfg::RW, QS = Cfg::QS, QKL = Cfg::QKL;
    // One value head per workgroup: the waves split the q/k prologue (one
    // barrier).  Several heads per workgroup (GQA groups): every wave runs the
    // whole q/k prologue itself, so no wave waits for another before its
    // state stream -- these launches run one workgroup per CU in many rounds,
    // where that wait is exposed.
    constexpr bool kSplit = GT == 1;
    extern __shared__ __attribute__((aligned(16))) float lds[];

    const int b = blockIdx.x / a.Hqk, kh = blockIdx.x % a.Hqk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // GT: heads per group fixed at compile time (1 or 2), or 0 = runtime a.G.
    const int G = GT ? GT : a.G;
    const int slot = a.slots[b];

    if (slot < 0 || slot >= a.num_rows) {  // skipped entry: zero outputs, no pool access
        for (int i = threadIdx.x; i < G * D; i += Cfg::NT)
            st<IOT>(a.out, ((int64_t)b * a.Hv + kh * G) * D + i, 0.f);
        return;
    }

    float *wq = kSplit ? lds : lds + wave * (2 * D + RW);  // q conv outputs
    float *wk = wq + D;                                     // k conv outputs
    float *wv = kSplit ? lds + 2 * D + wave * RW : wk + D;  // this wave's v band
    CT *cs = CONV ? static_cast<CT *>(a.conv_pool) + (int64_t)slot * a.conv_stride : nullptr;
    const int64_t xrow = (int64_t)b * a.C;
    const float bias_on = a.bias ? 1.f : 0.f;
    const int col0 = (lane % LPR) * EPL;
    const int rband = wave * RW;                  // first row of this wave's band
    const int cq0 = kh * D, ck0 = a.Hqk * D + kh * D;
    const int cv0 = 2 * a.Hqk * D + kh * G * D;   // first v channel of the group

    // ---- 1. prologue loads (small) ----
    // Split prologue: wave w convolves q channels QS w .. QS w + QS - 1 on
    // lanes 0..31 and the same k channels on lanes 32..63, so it alone reads
    // (and rolls) their conv history.  Whole prologue: lane l convolves q and
    // k channels l, l + 64, ..; the shared history is rolled at the end.
    // Indices are clamped instead of branched on, so every lane issues the
    // same loads and no control-flow join forces an early wait.
    const bool is_k = lane >= 32;
    const int qk_i = QS * wave + min(lane & 31, QS - 1);  // channel within the block
    const bool qk_on = (lane & 31) < QS;
    const int qk_c = (is_k ? ck0 : cq0) + qk_i;
    constexpr int NQK = kSplit ? 1 : QKL;
    ConvIn<IOT, CT> qi[NQK], ki[NQK], vi;
    if constexpr (kSplit) {
        load_conv_in<IOT, CT, CONV>(qi[0], a, cs, xrow, qk_c);
    } else {
#pragma unroll
        for (int t = 0; t < QKL; ++t) {
            const int i = min(lane + 64 * t, D - 1);
            load_conv_in<IOT, CT, CONV>(qi[t], a, cs, xrow, cq0 + i);
            load_conv_in<IOT, CT, CONV>(ki[t], a, cs, xrow, ck0 + i);
        }
    }
    const int vl = min(lane, RW - 1);  // this lane's v channel in the band
    load_conv_in<IOT, CT, CONV>(vi, a, cs, xrow, cv0 + rband + vl);
    float gl[EPL], beta;
    load_gates<D, ST, KDA>(gl, beta, a, b, kh * G, col0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. prologue compute, before any state row is requested ----
    if constexpr (kSplit) {
        if (qk_on) {
            (is_k ? wk : wq)[qk_i] = conv_out<CONV>(qi[0], bias_on);
            if constexpr (CONV) roll_history<IOT, CT>(qi[0], a, cs, qk_c);  // only this lane reads it
        }
    } else {
#pragma unroll
        for (int t = 0; t < QKL; ++t) {
            const int i = lane + 64 * t;
            if (i < D) {
                wq[i] = conv_out<CONV>(qi[t], bias_on);
                wk[i] = conv_out<CONV>(ki[t], bias_on);
            }
        }
    }
    if (lane < RW) {
        wv[lane] = conv_out<CONV>(vi, bias_on);
        if constexpr (CONV) roll_history<IOT, CT>(vi, a, cs, cv0 + rband + lane);  // only this wave reads it
    }
    if constexpr (kSplit) __syncthreads();  // every wave's q/k conv outputs written
    else __builtin_amdgcn_wave_barrier();   // this wave's LDS band written above, read below
    float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
    for (int t = 0; t < (D + 63) / 64; ++t) {
        const int i = lane + 64 * t;
        if (i < D) {
            const float yq = wq[i], yk = wk[i];
            sq = fmaf(yq, yq, sq);
            sk = fmaf(yk, yk, sk);
            sqk = fmaf(yq, yk, sqk);
        }
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    sqk = wave_sum(sqk);
    const float inv_q = 1.0f / sqrtf(sq + a.eps);
    const float inv_k = 1.0f / sqrtf(sk + a.eps);
    const float kq = sqk * inv_q * inv_k;
    float kk[EPL], qq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kk[e] = wk[col0 + e] * inv_k;
        qq[e] = wq[col0 + e] * inv_q;
    }

    // ---- 3. all state rows of the first head ----
    // Issued only now (kept below the prologue by the scheduling barriers):
    // with every workgroup's rows requested at once the small prologue loads
    // queue behind them, so each wave first finishes its prologue and then
    // streams its rows, consuming each as it lands.
    __builtin_amdgcn_sched_barrier(0);
    ST *S0 = static_cast<ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride +
             (int64_t)kh * G * D * D;
    uint4 buf[NJ];
    load_rows<D, ST>(buf, S0, wave, lane);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. the gated delta rule, head by head ----
    // Heads 0 .. G-2 prefetch the next head's rows and gates unconditionally
    // (a conditional prefetch would make the wait counts after it
    // conservative); the last head runs after the loop with nothing behind it.
    auto head = [&](int hg, const uint4 *rows, const float *glh, float bh) {
        const int h = kh * G + hg;
        ST *S = S0 + (int64_t)hg * D * D;
        float al[EPL], ak[EPL], aq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            al[e] = fast_exp(glh[e]);
            ak[e] = al[e] * kk[e];
            aq[e] = al[e] * qq[e];
        }
        float vrow[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int rr = j * RPW + lane / LPR;  // row inside the band
            vrow[j] = (D >= RPW || rr < RW) ? wv[rr] : 0.f;
        }
        float my_o = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (wave * NJ + j) * RPW + lane / LPR;
            float s[EPL];
            Stor<ST>::unpack(rows[j], s);
            float u = 0.f, p = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                u = fmaf(s[e], ak[e], u);
                p = fmaf(s[e], aq[e], p);
            }
            u = group_sum<LPR>(u);
            p = group_sum<LPR>(p);
            const float d = bh * (vrow[j] - u);
            const float o = a.scale * fmaf(d, kq, p);
            if (lane % LPR == j) my_o = o;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s[e] = fmaf(s[e], al[e], d * kk[e]);
            if (D >= RPW || r < D)
                st_stream(S + (int64_t)r * D + col0, Stor<ST>::pack(s));
        }
        // one output store per lane: lane (l % LPR == j) holds row instruction j
        const int j = lane % LPR;
        const int r = (wave * NJ + j) * RPW + lane / LPR;
        if (j < NJ && (D >= RPW || r < D))
            st<IOT>(a.out, ((int64_t)b * a.Hv + h) * D + r, my_o);
    };

    // Process head hg while head hg + 1 is in flight.
    auto step = [&](int hg) {
        uint4 nxt[NJ];
        ConvIn<IOT, CT> vn;
        float gn[EPL], bn;
        load_conv_in<IOT, CT, CONV>(vn, a, cs, xrow, cv0 + (hg + 1) * D + rband + vl);
        load_gates<D, ST, KDA>(gn, bn, a, b, kh * G + hg + 1, col0);
        load_rows<D, ST>(nxt, S0 + (int64_t)(hg + 1) * D * D, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        head(hg, buf, gl, beta);
        __builtin_amdgcn_wave_barrier();  // this head's v band fully read
        if (lane < RW) {
            wv[lane] = conv_out<CONV>(vn, bias_on);
            if constexpr (CONV)
                roll_history<IOT, CT>(vn, a, cs, cv0 + (hg + 1) * D + rband + lane);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < NJ; ++j) buf[j] = nxt[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) gl[e] = gn[e];
        beta = bn;
    };
    if constexpr (GT == 2) {
        step(0);  // straight-line code: no loop preheader flush of the counters
    } else if constexpr (GT == 0) {
        for (int hg = 0; hg + 1 < G; ++hg) step(hg);
    }
    head(G - 1, buf, gl, beta);

    // ---- 5. whole prologue: roll the shared q/k history once every wave
    //      has read it ----
    if constexpr (CONV && !kSplit) {
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < QKL; ++t) {
                const int i = lane + 64 * t;
                if (i < D) {
                    roll_history<IOT, CT>(qi[t], a, cs, cq0 + i);
                    roll_history<IOT, CT>(ki[t], a, cs, ck0 + i);
                }
            }
        }
    }
}


// Launch for one head dim: every dtype combination and mode is a separate
// instantiation, chosen here from the runtime codes.
template <int D, typename ST, typename IOT, typename CT, bool KDA, bool CONV>
inline hipError_t launch_decode_cfg(const DecodeArgs &a, hipStream_t stream)
{
    using Cfg = DecodeCfg<D, ST>;
    const size_t lds_split = (size_t)Cfg::LDS_SPLIT * sizeof(float);
    const size_t lds_whole = (size_t)Cfg::LDS_WHOLE * sizeof(float);
    const dim3 grid((unsigned)(a.B * a.Hqk)), block(Cfg::NT);
    if (a.G == 1)
        hipLaunchKernelGGL((decode_kernel<D, ST, IOT, CT, KDA, 1, CONV>), grid, block, lds_split,
                           stream, a);
    else if (a.G == 2)
        hipLaunchKernelGGL((decode_kernel<D, ST, IOT, CT, KDA, 2, CONV>), grid, block, lds_whole,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<D, ST, IOT, CT, KDA, 0, CONV>), grid, block, lds_whole,
                           stream, a);
    return hipGetLastError();
}

template <int D, typename ST, typename IOT, typename CT>
inline hipError_t launch_decode_modes(const DecodeArgs &a, bool kda, hipStream_t stream)
{
    const bool conv = a.w != nullptr;
    if (kda) return conv ? launch_decode_cfg<D, ST, IOT, CT, true, true>(a, stream)
                         : launch_decode_cfg<D, ST, IOT, CT, true, false>(a, stream);
    return conv ? launch_decode_cfg<D, ST, IOT, CT, false, true>(a, stream)
                : launch_decode_cfg<D, ST, IOT, CT, false, false>(a, stream);
}

template <int D>
hipError_t launch_decode_dim(const DecodeArgs &a, int state_dtype, bool kda, hipStream_t stream)
{
    const int code = (state_dtype ? 4 : 0) | (a.io_dtype ? 2 : 0) | (a.conv_dtype ? 1 : 0);
    switch (code) {
    case 0: return launch_decode_modes<D, float, float, float>(a, kda, stream);
    case 1: return launch_decode_modes<D, float, float, bf16_t>(a, kda, stream);
    case 2: return launch_decode_modes<D, float, bf16_t, float>(a, kda, stream);
    case 3: return launch_decode_modes<D, float, bf16_t, bf16_t>(a, kda, stream);
    case 4: return launch_decode_modes<D, bf16_t, float, float>(a, kda, stream);
    case 5: return launch_decode_modes<D, bf16_t, float, bf16_t>(a, kda, stream);
    case 6: return launch_decode_modes<D, bf16_t, bf16_t, float>(a, kda, stream);
    default: return launch_decode_modes<D, bf16_t, bf16_t, bf16_t>(a, kda, stream);
    }
}

}  // namespace la
