// decode.hip -- fused single-token decode of Kimi Delta Attention (per-key-
// channel decay) and Gated DeltaNet (per-head scalar decay) on gfx950.
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
// G = H_v / H_qk value heads that share that q/k head.  Owning the whole
// group makes the workgroup the only reader and writer of every conv-state
// channel it touches (q, k and its v channels), so the in-place history roll
// needs no cross-workgroup ordering.
//
// State streaming.  Row i of a head's state (d_k contiguous) is split over
// LPR lanes holding 16 bytes each (8 bf16 or 4 fp32), so one wave instruction
// moves RPW = 64 / LPR consecutive rows = 1 KB contiguous: fully coalesced.
// Both row reductions (S'k and S'q) come out of one pass over the registers
// (DPP inside the LPR-lane group, bit-identical in every lane), the update is
// applied in registers and the row is stored back: the state crosses HBM once
// each way.  The state loads of the first head are issued before the conv
// prologue so the prologue's latency hides under them; with G > 1 the next
// head's rows are prefetched while the current head computes.
#include "la_device.h"
#include "la_internal.h"

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
    static_assert(LPR >= 1 && LPR <= 32, "row must fit in half a wave");
    static_assert(RI % NW == 0, "rows must split evenly over waves");
};

template <int D, typename ST>
__device__ __forceinline__ void load_head_rows(uint4 *buf, const ST *S, int wave, int lane)
{
    using Cfg = DecodeCfg<D, ST>;
    const int col0 = (lane % Cfg::LPR) * Cfg::EPL;
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j) {
        const int r = (wave * Cfg::NJ + j) * Cfg::RPW + lane / Cfg::LPR;
        if (D >= Cfg::RPW || r < D)
            buf[j] = *reinterpret_cast<const uint4 *>(S + (int64_t)r * D + col0);
        else
            buf[j] = make_uint4(0, 0, 0, 0);
    }
}

template <int D, typename ST, bool KDA>
__global__ void __launch_bounds__((DecodeCfg<D, ST>::NT)) decode_kernel(DecodeArgs a)
{
    using Cfg = DecodeCfg<D, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ;
    extern __shared__ float ys[];  // post-conv [q (D) | k (D) | v (G*D)]

    const int b = blockIdx.x / a.Hqk, kh = blockIdx.x % a.Hqk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.G, C = a.C;
    const int slot = a.slots[b];

    if (slot < 0 || slot >= a.num_rows) {  // skipped entry: zero outputs, no pool access
        for (int i = tid; i < G * D; i += Cfg::NT)
            store_elem(a.out, ((int64_t)b * a.Hv + kh * G) * D + i, a.io_dtype, 0.f);
        return;
    }

    // Issue the first head's state loads before anything else.
    ST *S0 = static_cast<ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride +
             (int64_t)kh * G * D * D;
    uint4 buf[NJ];
    load_head_rows<D, ST>(buf, S0, wave, lane);

    // ---- prologue: short conv + SiLU for the group's q, k, v channels ----
    const int nch = (2 + G) * D;
    const int64_t xrow = (int64_t)b * C;
    const int csz = a.conv_dtype ? 2 : 4;
    char *cs = a.w ? static_cast<char *>(a.conv_pool) + (int64_t)slot * a.conv_stride * csz
                   : nullptr;
    for (int j = tid; j < nch; j += Cfg::NT) {
        int c;
        if (j < D) c = kh * D + j;
        else if (j < 2 * D) c = a.Hqk * D + kh * D + (j - D);
        else c = 2 * a.Hqk * D + kh * G * D + (j - 2 * D);
        const float xv = load_elem(a.x, xrow + c, a.io_dtype);
        float y = xv;
        if (a.w) {
            const float h0 = load_elem(cs, c, a.conv_dtype);
            const float h1 = load_elem(cs, C + c, a.conv_dtype);
            const float h2 = load_elem(cs, 2 * C + c, a.conv_dtype);
            const float4 wc = reinterpret_cast<const float4 *>(a.w)[c];
            float acc = a.bias ? a.bias[c] : 0.f;
            acc = fmaf(wc.x, h0, acc);
            acc = fmaf(wc.y, h1, acc);
            acc = fmaf(wc.z, h2, acc);
            acc = fmaf(wc.w, xv, acc);
            y = silu(acc);
            // Roll the history: rows 1, 2 move to 0, 1 and the input becomes
            // row 2.  fp32 <-> bf16 round trips are exact, so this is a bit
            // copy whenever the dtypes agree.
            store_elem(cs, c, a.conv_dtype, h1);
            store_elem(cs, C + c, a.conv_dtype, h2);
            store_elem(cs, 2 * C + c, a.conv_dtype, xv);
        }
        ys[j] = y;
    }
    __syncthreads();

    // ---- L2 norms of q and k and their dot product (every wave, same order) --
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    for (int i = lane; i < D; i += 64) {
        const float qv = ys[i], kv = ys[D + i];
        sq = fmaf(qv, qv, sq);
        sk = fmaf(kv, kv, sk);
        sqk = fmaf(qv, kv, sqk);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    sqk = wave_sum(sqk);
    const float inv_q = 1.0f / sqrtf(sq + a.eps);
    const float inv_k = 1.0f / sqrtf(sk + a.eps);
    const float kq = sqk * inv_q * inv_k;

    const int col0 = (lane % LPR) * EPL;
    float kk[EPL], qq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kk[e] = ys[D + col0 + e] * inv_k;
        qq[e] = ys[col0 + e] * inv_q;
    }

    // ---- the gated delta rule, head by head ----
    for (int hg = 0; hg < G; ++hg) {
        const int h = kh * G + hg;
        ST *S = S0 + (int64_t)hg * D * D;
        uint4 nxt[NJ];
        if (hg + 1 < G) load_head_rows<D, ST>(nxt, S + D * D, wave, lane);

        float al[EPL];
        if constexpr (KDA) {
            const float *gp = a.g + ((int64_t)b * a.Hv + h) * D + col0;
#pragma unroll
            for (int e = 0; e < EPL; e += 4) {
                const float4 g4 = *reinterpret_cast<const float4 *>(gp + e);
                al[e] = expf(g4.x); al[e + 1] = expf(g4.y);
                al[e + 2] = expf(g4.z); al[e + 3] = expf(g4.w);
            }
        } else {
            const float a1 = expf(a.g[(int64_t)b * a.Hv + h]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) al[e] = a1;
        }
        float ak[EPL], aq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            ak[e] = al[e] * kk[e];
            aq[e] = al[e] * qq[e];
        }
        const float beta = a.beta[(int64_t)b * a.Hv + h];
        const float *vs = ys + 2 * D + hg * D;
        const int64_t obase = ((int64_t)b * a.Hv + h) * D;

#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (wave * NJ + j) * RPW + lane / LPR;
            const bool row_ok = D >= RPW || r < D;
            float s[EPL];
            Stor<ST>::unpack(buf[j], s);
            float u = 0.f, p = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                u = fmaf(s[e], ak[e], u);
                p = fmaf(s[e], aq[e], p);
            }
            u = group_sum<LPR>(u);
            p = group_sum<LPR>(p);
            const float vv = row_ok ? vs[r] : 0.f;
            const float d = beta * (vv - u);
            const float o = a.scale * fmaf(d, kq, p);
#pragma unroll
            for (int e = 0; e < EPL; ++e) s[e] = fmaf(s[e], al[e], d * kk[e]);
            if (row_ok) {
                *reinterpret_cast<uint4 *>(S + (int64_t)r * D + col0) = Stor<ST>::pack(s);
                if (lane % LPR == 0) store_elem(a.out, obase + r, a.io_dtype, o);
            }
        }
        if (hg + 1 < G) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) buf[j] = nxt[j];
        }
    }
}

template <int D, typename ST, bool KDA>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream)
{
    using Cfg = DecodeCfg<D, ST>;
    const size_t lds = (size_t)(2 + a.G) * D * sizeof(float);
    hipLaunchKernelGGL((decode_kernel<D, ST, KDA>), dim3((unsigned)(a.B * a.Hqk)),
                       dim3(Cfg::NT), lds, stream, a);
    return hipGetLastError();
}

template <typename ST, bool KDA>
static hipError_t launch_decode_d(const DecodeArgs &a, int D, hipStream_t stream)
{
    switch (D) {
    case 16: return launch_decode_t<16, ST, KDA>(a, stream);
    case 32: return launch_decode_t<32, ST, KDA>(a, stream);
    case 64: return launch_decode_t<64, ST, KDA>(a, stream);
    case 128: return launch_decode_t<128, ST, KDA>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, int D, int state_dtype, bool kda,
                         hipStream_t stream)
{
    if (state_dtype) return kda ? launch_decode_d<bf16_t, true>(a, D, stream)
                                : launch_decode_d<bf16_t, false>(a, D, stream);
    return kda ? launch_decode_d<float, true>(a, D, stream)
               : launch_decode_d<float, false>(a, D, stream);
}

}  // namespace la
