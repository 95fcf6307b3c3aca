// spec.hip -- speculative decode on the recurrent state: multi-token verify,
// exact commit, the conv-window scatter and the state-tracking copy.
//
// What they compute (the ReplaySSM passages of xxmr.cn/news/181459):
//   verify  -- up to D draft tokens per request run through the short conv
//              and the gated delta rule from the pool checkpoint; every step's
//              output is produced, the state is carried across the tokens and
//              never written back, and each step's record (d, k, g, rawv,
//              rawk, beta) is appended to a per-slot ring of depth L, together
//              with the conv history after each step (the per-step conv
//              window of that page's "intermediate_conv_window" passage);
//   commit  -- the accepted prefix is replayed from the checkpoint with
//              k = rawk / sqrt(|rawk|^2 + eps), alpha = exp(g),
//              S <- S Diag(alpha), d = beta (rawv - S k), S <- S + d k^T,
//              and the result is stored back;
//   scatter -- the conv history of the last accepted step is written to the
//              persistent conv state, under a mask;
//   track   -- the conv and SSM rows of an active slot are copied to a
//              tracking slot, under a mask (that page's state-tracking
//              passage);
//   fold    -- the fast rebuild: the state after m ring steps from the
//              checkpoint and the steps' (d, k, g) by the unrolled sum, with
//              no replay of the delta rule (that page's d/k/g passage).
// The conv output is rounded to the I/O dtype before the recurrence, as a
// separate conv kernel's output tensor would be, so the ring holds exactly the
// values verify used and the commit reproduces verify's arithmetic: both
// kernels run the same per-row update code.
//
// Work decomposition of verify and commit: one workgroup per (request, value
// head), the head's state rows spread over the waves as in the decode kernel
// (16-byte lane chunks, LPR lanes per row), held in fp32 registers across the
// steps.  Verify forms a chunk's q|k|v conv outputs, decays, norms and ring
// records up front, so its steps only update the state rows, with no barrier
// between steps.  Both kernels first stage
// the inputs of up to eight steps in LDS (verify: the pre-conv inputs of the
// head's channels and the gates; commit: the ring records), with every load
// issued back to back, so a step waits for memory once per eight steps.
#include "decode_kernel.h"
#include "la_device.h"
#include "la_internal.h"

namespace la {

namespace {

constexpr int HD = 128;     // head dim of the speculative kernels (d_k = d_v)
constexpr int kChunk = 8;   // steps whose inputs are staged in LDS at once

template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16_t>(float v)
{
    return bf16_to_f32(f32_to_bf16(v));
}

__device__ __forceinline__ int64_t ring_at(int slot, int Hv, int L, int h, int pos, int n)
{
    return (((int64_t)slot * Hv + h) * L + pos) * n;
}

// The shared per-row step:  s <- s Diag(al);  u = s . kk;  d = beta (v - u);
// s <- s + d kk.  Returns d (identical in every lane of the row's group).
template <int EPL, int LPR>
__device__ __forceinline__ float row_step(float (&s)[EPL], const float (&al)[EPL],
                                          const float (&kk)[EPL], float v, float beta)
{
    float u = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        s[e] *= al[e];
        u = fmaf(s[e], kk[e], u);
    }
    u = group_sum<LPR>(u);
    const float d = beta * (v - u);
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = fmaf(d, kk[e], s[e]);
    return d;
}

// 1 / sqrt(|x|^2 + eps) of a 128-vector held as lane, lane + 64 (wave-wide).
__device__ __forceinline__ float inv_norm128(float x0, float x1, float eps)
{
    return 1.0f / sqrtf(wave_sum(fmaf(x1, x1, x0 * x0)) + eps);
}

// ---------------------------------------------------------------------------
// verify
// ---------------------------------------------------------------------------
template <typename ST, typename IOT, typename CT, bool KDA, bool CONV>
__global__ void __launch_bounds__((DecodeCfg<HD, ST>::NT)) verify_kernel(VerifyArgs a)
{
    using Cfg = DecodeCfg<HD, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = Cfg::NT;
    constexpr int NCH = 3 * HD;                // the head's q, k, v channels
    constexpr int CPT = (NCH + NT - 1) / NT;   // channels per thread
    constexpr int XPT = (kChunk * NCH + NT - 1) / NT;  // staged inputs per thread
    constexpr int GPT = (kChunk * HD + NT - 1) / NT;   // staged gates per thread
    __shared__ float xs[kChunk][NCH];          // the chunk's pre-conv inputs, then its q|k|v
    __shared__ float nq[kChunk], nk[kChunk];   // the chunk's inverse q and k norms
    __shared__ float gs[kChunk][HD];           // the chunk's log-decays, then exp of them (GDN: broadcast)
    __shared__ float bs[kChunk];               // the chunk's betas

    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv, kh = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = a.slots[b];
    const int n = min(max(a.n_tok[b], 0), a.D);
    auto out_at = [&](int t, int i) { return (((int64_t)b * a.D + t) * a.Hv + h) * HD + i; };
    const int first_zero = (slot < 0 || slot >= a.num_rows) ? 0 : n;
    for (int i = tid + first_zero * HD; i < a.D * HD; i += NT)  // steps past n (or a skipped entry)
        st<IOT>(a.out, out_at(i / HD, i % HD), 0.f);
    if (first_zero == 0) return;

    // The local channel j (over [q | k | v] of this head) -> global channel.
    auto glob = [&](int j) {
        return j < HD ? kh * HD + j
             : j < 2 * HD ? a.Hqk * HD + kh * HD + (j - HD) : 2 * a.Hqk * HD + h * HD + (j - 2 * HD);
    };
    // The conv history of the channels this thread owns (local index
    // j = tid + NT m), carried across the steps.  Everything else about a
    // channel (its global index, weights, bias) is re-derived in each chunk,
    // so only the history stays live across chunks.
    float h0[CPT], h1[CPT], h2[CPT];
    if constexpr (CONV) {
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const int64_t c = (int64_t)slot * a.conv_stride + glob(min(tid + NT * m, NCH - 1));
            h0[m] = ld<CT>(a.conv_pool, c);
            h1[m] = ld<CT>(a.conv_pool, c + a.C);
            h2[m] = ld<CT>(a.conv_pool, c + 2 * a.C);
        }
    }

    // The head's state rows, unpacked to fp32 registers for the whole call.
    const ST *S = static_cast<const ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride +
                  (int64_t)h * HD * HD;
    float s[NJ][EPL];
    {
        uint4 raw[NJ];
        load_rows<HD, ST>(raw, S, wave, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) Stor<ST>::unpack(raw[j], s[j]);
    }
    const int col0 = (lane % LPR) * EPL;
    const RingArgs &R = a.ring;

    for (int t0 = 0; t0 < n; t0 += kChunk) {
    // ---- stage the chunk's inputs and gates in LDS: every load issued back to
    //      back (indices clamped into the chunk, so no branch around a load).
    //      The staging indices are re-derived from an opaque copy of the
    //      thread id in each chunk, so they are not kept live across chunks.
    const int nc = min(kChunk, n - t0);
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    float4 wc[CPT];
    float bias[CPT];
    {
        float xv[XPT], gv2[GPT], bv = 0.f;
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int i = min(ltid + q * NT, kChunk * NCH - 1);
            const int tt = min(i / NCH, nc - 1);
            xv[q] = ld<IOT>(a.x, ((int64_t)b * a.D + t0 + tt) * a.C + glob(i % NCH));
        }
#pragma unroll
        for (int q = 0; q < GPT; ++q) {
            const int i = min(ltid + q * NT, kChunk * HD - 1);
            const int64_t bt = (int64_t)b * a.D + t0 + min(i / HD, nc - 1);
            gv2[q] = KDA ? a.g[(bt * a.Hv + h) * HD + i % HD] : a.g[bt * a.Hv + h];
        }
        if (tid < kChunk) bv = a.beta[((int64_t)b * a.D + t0 + min(tid, nc - 1)) * a.Hv + h];
        if constexpr (CONV) {
#pragma unroll
            for (int m = 0; m < CPT; ++m) {
                const int gc = glob(min(ltid + NT * m, NCH - 1));
                wc[m] = reinterpret_cast<const float4 *>(a.w)[gc];
                bias[m] = a.bias ? a.bias[gc] : 0.f;
            }
        }
        __syncthreads();  // the previous chunk's staged values are no longer read
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int i = tid + q * NT;
            if (i < kChunk * NCH) xs[i / NCH][i % NCH] = xv[q];
        }
#pragma unroll
        for (int q = 0; q < GPT; ++q) {
            const int i = tid + q * NT;
            if (i < kChunk * HD) gs[i / HD][i % HD] = gv2[q];
        }
        if (tid < kChunk) bs[tid] = bv;
        __syncthreads();
    }
    // ---- the chunk's conv outputs (rounded to the I/O dtype, in place over
    //      the staged inputs), its decays alpha = exp(g) (in place over the
    //      gates) and its ring records, before any state row is touched: the
    //      conv history of each owned channel steps through the chunk in
    //      registers
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
        const int j = ltid + NT * m;
        if (j >= NCH) continue;
        const int gc = glob(j);
        // q/k windows are written by the first value head of the group only
        const bool win_out = j >= 2 * HD || h % a.G == 0;
        for (int tt = 0; tt < nc; ++tt) {
            const int t = t0 + tt;
            const int pos = (a.ring_base[b] + t) & (R.L - 1);
            const int64_t bt = (int64_t)b * a.D + t;
            const float x = xs[tt][j];
            float y = x;
            if constexpr (CONV) {
                float acc = bias[m];
                acc = fmaf(wc[m].x, h0[m], acc);
                acc = fmaf(wc[m].y, h1[m], acc);
                acc = fmaf(wc[m].z, h2[m], acc);
                acc = fmaf(wc[m].w, x, acc);
                y = silu(acc);
                h0[m] = h1[m];
                h1[m] = h2[m];
                h2[m] = round_to<CT>(x);
                if (win_out) {
                    const int64_t wrow = bt * 3 * a.C + gc;
                    st<CT>(a.windows, wrow, h0[m]);
                    st<CT>(a.windows, wrow + a.C, h1[m]);
                    st<CT>(a.windows, wrow + 2 * a.C, h2[m]);
                }
            }
            y = round_to<IOT>(y);
            xs[tt][j] = y;
            if (j >= 2 * HD) st<IOT>(R.rawv, ring_at(slot, a.Hv, R.L, h, pos, HD) + (j - 2 * HD), y);
            else if (j >= HD) st<IOT>(R.rawk, ring_at(slot, a.Hv, R.L, h, pos, HD) + (j - HD), y);
        }
    }
    for (int i = tid; i < nc * HD; i += NT) {
        const int tt = i / HD, c = i % HD;
        const int pos = (a.ring_base[b] + t0 + tt) & (R.L - 1);
        const float g = gs[tt][c];
        if constexpr (KDA) R.g[ring_at(slot, a.Hv, R.L, h, pos, HD) + c] = g;
        else if (c == 0) R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)] = g;
        if (c == 0) R.beta[ring_at(slot, a.Hv, R.L, h, pos, 1)] = bs[tt];
        gs[tt][c] = fast_exp(g);
    }
    __syncthreads();  // the chunk's q|k|v and decays complete
    // ---- the steps' norms, wave w taking steps w, w + NW, ..; normalised k
    //      to the ring
    for (int tt = wave; tt < nc; tt += Cfg::NW) {
        const int pos = (a.ring_base[b] + t0 + tt) & (R.L - 1);
        const float q0 = xs[tt][lane], q1 = xs[tt][lane + 64];
        const float k0 = xs[tt][HD + lane], k1 = xs[tt][HD + lane + 64];
        const float inv_q = inv_norm128(q0, q1, a.eps);
        const float inv_k = inv_norm128(k0, k1, a.eps);
        if (lane == 0) {
            nq[tt] = inv_q;
            nk[tt] = inv_k;
        }
        const int64_t kr = ring_at(slot, a.Hv, R.L, h, pos, HD);
        st<IOT>(R.k, kr + lane, k0 * inv_k);
        st<IOT>(R.k, kr + lane + 64, k1 * inv_k);
    }
    __syncthreads();
    // ---- the steps: only the state rows, with no barrier between steps
    for (int tt = 0; tt < nc; ++tt) {
        const int t = t0 + tt;
        const int pos = (a.ring_base[b] + t) & (R.L - 1);
        const float inv_q = nq[tt], inv_k = nk[tt];
        float kk[EPL], qq[EPL], al[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kk[e] = xs[tt][HD + col0 + e] * inv_k;
            qq[e] = xs[tt][col0 + e] * inv_q;
            al[e] = gs[tt][col0 + e];
        }
        const float beta = bs[tt];
        // every lane of a row group gets the row's sums; lane (l % LPR == j)
        // keeps row instruction j's, so each lane stores once per step
        float my_o = 0.f, my_d = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (wave * NJ + j) * RPW + lane / LPR;
            const float d = row_step<EPL, LPR>(s[j], al, kk, xs[tt][2 * HD + r], beta);
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) p = fmaf(s[j][e], qq[e], p);
            p = group_sum<LPR>(p);
            if (lane % LPR == j) {
                my_o = p;
                my_d = d;
            }
        }
        const int jl = lane % LPR, r = (wave * NJ + jl) * RPW + lane / LPR;
        if (jl < NJ) {
            st<IOT>(a.out, out_at(t, r), a.scale * my_o);
            st<IOT>(R.d, ring_at(slot, a.Hv, R.L, h, pos, HD) + r, my_d);
        }
    }
    }
}

// ---------------------------------------------------------------------------
// commit
// ---------------------------------------------------------------------------
template <typename ST, typename IOT, bool KDA>
__global__ void __launch_bounds__((DecodeCfg<HD, ST>::NT)) commit_kernel(CommitArgs a)
{
    using Cfg = DecodeCfg<HD, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = Cfg::NT;
    constexpr int VPT = (kChunk * HD + NT - 1) / NT;  // staged ring values per thread
    __shared__ float ks[kChunk][HD], vs[kChunk][HD], gsh[kChunk][HD], bsh[kChunk], nk[kChunk];
    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = a.slots[b];
    const int na = min(a.accepted[b], a.ring.L);
    if (slot < 0 || slot >= a.num_rows || na <= 0) return;  // nothing accepted: row unchanged

    ST *S = static_cast<ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride + (int64_t)h * HD * HD;
    float s[NJ][EPL];
    {
        uint4 raw[NJ];
        load_rows<HD, ST>(raw, S, wave, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) Stor<ST>::unpack(raw[j], s[j]);
    }
    const int col0 = (lane % LPR) * EPL;
    const RingArgs &R = a.ring;
    for (int t0 = 0; t0 < na; t0 += kChunk) {
        // stage the chunk's ring records in LDS, all loads back to back
        const int nc = min(kChunk, na - t0);
        float kv[VPT], vv[VPT], gv[VPT], bv = 0.f;
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int i = min(tid + q * NT, kChunk * HD - 1);
            const int pos = (a.ring_base[b] + t0 + min(i / HD, nc - 1)) & (R.L - 1);
            const int64_t vr = ring_at(slot, a.Hv, R.L, h, pos, HD) + i % HD;
            kv[q] = ld<IOT>(R.rawk, vr);
            vv[q] = ld<IOT>(R.rawv, vr);
            gv[q] = KDA ? R.g[vr] : R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)];
        }
        if (tid < kChunk) {
            const int pos = (a.ring_base[b] + t0 + min(tid, nc - 1)) & (R.L - 1);
            bv = R.beta[ring_at(slot, a.Hv, R.L, h, pos, 1)];
        }
        __syncthreads();  // the previous chunk's records are no longer read
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int i = tid + q * NT;
            if (i < kChunk * HD) {
                ks[i / HD][i % HD] = kv[q];
                vs[i / HD][i % HD] = vv[q];
                gsh[i / HD][i % HD] = gv[q];
            }
        }
        if (tid < kChunk) bsh[tid] = bv;
        __syncthreads();
        // the chunk's inverse k norms (wave w: steps w, w + NW, ..) and its
        // decays alpha = exp(g) (in place), formed once for all rows
        for (int tt = wave; tt < nc; tt += Cfg::NW) {
            const float inv_k = inv_norm128(ks[tt][lane], ks[tt][lane + 64], a.eps);
            if (lane == 0) nk[tt] = inv_k;
        }
        for (int i = tid; i < nc * HD; i += NT) gsh[i / HD][i % HD] = fast_exp(gsh[i / HD][i % HD]);
        __syncthreads();
        for (int tt = 0; tt < nc; ++tt) {
            const float inv_k = nk[tt];
            float kk[EPL], al[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kk[e] = ks[tt][col0 + e] * inv_k;
                al[e] = gsh[tt][col0 + e];
            }
            const float beta = bsh[tt];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = (wave * NJ + j) * RPW + lane / LPR;
                row_step<EPL, LPR>(s[j], al, kk, vs[tt][r], beta);
            }
        }
    }
    const int c0 = col0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = (wave * NJ + j) * RPW + lane / LPR;
        st_stream(S + (int64_t)r * HD + c0, Stor<ST>::pack(s[j]));
    }
}

// ---------------------------------------------------------------------------
// fast rebuild (ring fold)
// ---------------------------------------------------------------------------
// S_m = S_0 Diag(exp(G_m)) + sum_j d_j (k_j . exp(G_m - G_j))^T with G_j the
// cumulative log decay of the first j folded steps: the unrolled sum of the
// ReplaySSM d/k/g passage, 16 steps per LDS pass (passes compose).
constexpr int kFold = 16;
template <typename ST, typename IOT, bool KDA, bool PROJ>
__global__ void __launch_bounds__((DecodeCfg<HD, ST>::NT)) fold_kernel(FoldArgs a)
{
    using Cfg = DecodeCfg<HD, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = Cfg::NT;
    constexpr int VPT = (kFold * HD + NT - 1) / NT;
    __shared__ float dsh[kFold][HD];  // d_j
    __shared__ float esh[kFold][HD];  // k_j, then k_j exp(G_end - G_j)
    __shared__ float gsh[kFold][HD];  // g_j, then G_j
    __shared__ float eend[HD];        // exp(G_end)
    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = a.slots[b], dst = a.dst ? a.dst[b] : slot;
    if (slot < 0 || slot >= a.num_rows || dst < 0 || dst >= a.num_rows) {
        if constexpr (PROJ)
            for (int i = tid; i < HD; i += NT) st<IOT>(a.out, ((int64_t)b * a.Hv + h) * HD + i, 0.f);
        return;
    }
    const int m = min(max(a.m[b], 0), a.ring.L);
    const ST *S0 = static_cast<const ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride +
                   (int64_t)h * HD * HD;
    float s[NJ][EPL];
    {
        uint4 raw[NJ];
        load_rows<HD, ST>(raw, S0, wave, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) Stor<ST>::unpack(raw[j], s[j]);
    }
    const int col0 = (lane % LPR) * EPL;
    const RingArgs &R = a.ring;
    for (int t0 = 0; t0 < m; t0 += kFold) {
        const int nc = min(kFold, m - t0);
        float dv_[VPT], kv[VPT], gv[VPT];
#pragma unroll
        for (int q = 0; q < VPT; ++q) {  // clamped indices: every load issued, no branch
            const int i = min(tid + q * NT, kFold * HD - 1);
            const int pos = (a.ring_base[b] + t0 + min(i / HD, nc - 1)) & (R.L - 1);
            const int64_t vr = ring_at(slot, a.Hv, R.L, h, pos, HD) + i % HD;
            dv_[q] = ld<IOT>(R.d, vr);
            kv[q] = ld<IOT>(R.k, vr);
            gv[q] = KDA ? R.g[vr] : R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)];
        }
        __syncthreads();  // the previous pass's tables are no longer read
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int i = tid + q * NT;
            if (i < kFold * HD) {
                dsh[i / HD][i % HD] = dv_[q];
                esh[i / HD][i % HD] = kv[q];
                gsh[i / HD][i % HD] = gv[q];
            }
        }
        __syncthreads();
        if (tid < HD) {  // per channel: cumulative decay, then the decayed keys
            float G = 0.f;
            for (int t = 0; t < nc; ++t) {
                G += gsh[t][tid];
                gsh[t][tid] = G;
            }
            eend[tid] = fast_exp(G);
            for (int t = 0; t < nc; ++t) esh[t][tid] *= fast_exp(G - gsh[t][tid]);
        }
        __syncthreads();
        float ee[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) ee[e] = eend[col0 + e];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e) s[j][e] *= ee[e];
        for (int t = 0; t < nc; ++t) {
            float kt[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) kt[e] = esh[t][col0 + e];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float dt = dsh[t][(wave * NJ + j) * RPW + lane / LPR];
#pragma unroll
                for (int e = 0; e < EPL; ++e) s[j][e] = fmaf(dt, kt[e], s[j][e]);
            }
        }
    }
    ST *Sd = static_cast<ST *>(a.ssm_pool) + (int64_t)dst * a.ssm_stride + (int64_t)h * HD * HD;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = (wave * NJ + j) * RPW + lane / LPR;
        st_stream(Sd + (int64_t)r * HD + col0, Stor<ST>::pack(s[j]));
    }
    if constexpr (PROJ) {
        const int64_t qb = ((int64_t)b * a.Hv + h) * HD;
        const float inv_q = inv_norm128(ld<IOT>(a.q, qb + lane), ld<IOT>(a.q, qb + lane + 64), a.eps);
        float qq[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) qq[e] = ld<IOT>(a.q, qb + col0 + e) * inv_q;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) p = fmaf(s[j][e], qq[e], p);
            p = group_sum<LPR>(p);
            if (lane % LPR == 0) st<IOT>(a.out, qb + (wave * NJ + j) * RPW + lane / LPR, a.scale * p);
        }
    }
}

// ---------------------------------------------------------------------------
// conv-window scatter and state-tracking copy: 16-byte copies
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) conv_scatter_kernel(ScatterArgs a)
{
    const int b = blockIdx.y;
    if (a.mask && !a.mask[b]) return;
    const int step = a.step[b], slot = a.slots[b];
    if (step < 0 || step >= a.D || slot < 0 || slot >= a.num_rows) return;
    const int es = a.conv_dtype ? 2 : 4;
    const int64_t units = (int64_t)3 * a.C * es / 16;
    const char *src = static_cast<const char *>(a.windows) + ((int64_t)b * a.D + step) * 3 * a.C * es;
    char *dst = static_cast<char *>(a.conv_pool) + (int64_t)slot * a.conv_stride * es;
    for (int64_t u = blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256)
        reinterpret_cast<uint4 *>(dst)[u] = reinterpret_cast<const uint4 *>(src)[u];
}

__global__ void __launch_bounds__(256) track_copy_kernel(TrackArgs a)
{
    const int b = blockIdx.y;
    if (a.mask && !a.mask[b]) return;
    const int src = a.src[b], dst = a.dst[b];
    if (src < 0 || src >= a.num_rows || dst < 0 || dst >= a.num_rows || src == dst) return;
    const int64_t su = a.ssm_row_b / 16, cu = a.conv_row_b / 16;
    for (int64_t u = blockIdx.x * 256 + threadIdx.x; u < su + cu; u += (int64_t)gridDim.x * 256) {
        if (u < su) {
            const uint4 v = ld_stream(a.ssm_pool + src * a.ssm_stride_b + 16 * u);
            st_stream(a.ssm_pool + dst * a.ssm_stride_b + 16 * u, v);
        } else {
            const int64_t c = u - su;
            const uint4 v = ld_stream(a.conv_pool + src * a.conv_stride_b + 16 * c);
            st_stream(a.conv_pool + dst * a.conv_stride_b + 16 * c, v);
        }
    }
}

template <typename ST, typename IOT, typename CT, bool KDA>
hipError_t launch_verify_t(const VerifyArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.B * a.Hv)), block(DecodeCfg<HD, ST>::NT);
    if (a.w)
        hipLaunchKernelGGL((verify_kernel<ST, IOT, CT, KDA, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((verify_kernel<ST, IOT, CT, KDA, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <typename ST, typename IOT, typename CT>
hipError_t launch_verify_k(const VerifyArgs &a, bool kda, hipStream_t stream)
{
    return kda ? launch_verify_t<ST, IOT, CT, true>(a, stream)
               : launch_verify_t<ST, IOT, CT, false>(a, stream);
}

template <typename ST, typename IOT, bool KDA>
hipError_t launch_commit_t(const CommitArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((commit_kernel<ST, IOT, KDA>), dim3((unsigned)(a.B * a.Hv)),
                       dim3(DecodeCfg<HD, ST>::NT), 0, stream, a);
    return hipGetLastError();
}

template <typename ST, typename IOT, bool KDA>
hipError_t launch_fold_t(const FoldArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.B * a.Hv)), block(DecodeCfg<HD, ST>::NT);
    if (a.q)
        hipLaunchKernelGGL((fold_kernel<ST, IOT, KDA, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((fold_kernel<ST, IOT, KDA, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fold(const FoldArgs &a, int state_dtype, bool kda, hipStream_t stream)
{
    const int code = (state_dtype ? 2 : 0) | (a.io_dtype ? 1 : 0);
    switch (code) {
    case 0: return kda ? launch_fold_t<float, float, true>(a, stream)
                       : launch_fold_t<float, float, false>(a, stream);
    case 1: return kda ? launch_fold_t<float, bf16_t, true>(a, stream)
                       : launch_fold_t<float, bf16_t, false>(a, stream);
    case 2: return kda ? launch_fold_t<bf16_t, float, true>(a, stream)
                       : launch_fold_t<bf16_t, float, false>(a, stream);
    default: return kda ? launch_fold_t<bf16_t, bf16_t, true>(a, stream)
                        : launch_fold_t<bf16_t, bf16_t, false>(a, stream);
    }
}

hipError_t launch_verify(const VerifyArgs &a, int state_dtype, bool kda, hipStream_t stream)
{
    const int code = (state_dtype ? 4 : 0) | (a.io_dtype ? 2 : 0) | (a.conv_dtype ? 1 : 0);
    switch (code) {
    case 0: return launch_verify_k<float, float, float>(a, kda, stream);
    case 1: return launch_verify_k<float, float, bf16_t>(a, kda, stream);
    case 2: return launch_verify_k<float, bf16_t, float>(a, kda, stream);
    case 3: return launch_verify_k<float, bf16_t, bf16_t>(a, kda, stream);
    case 4: return launch_verify_k<bf16_t, float, float>(a, kda, stream);
    case 5: return launch_verify_k<bf16_t, float, bf16_t>(a, kda, stream);
    case 6: return launch_verify_k<bf16_t, bf16_t, float>(a, kda, stream);
    default: return launch_verify_k<bf16_t, bf16_t, bf16_t>(a, kda, stream);
    }
}

hipError_t launch_commit(const CommitArgs &a, int state_dtype, bool kda, hipStream_t stream)
{
    const int code = (state_dtype ? 2 : 0) | (a.io_dtype ? 1 : 0);
    switch (code) {
    case 0: return kda ? launch_commit_t<float, float, true>(a, stream)
                       : launch_commit_t<float, float, false>(a, stream);
    case 1: return kda ? launch_commit_t<float, bf16_t, true>(a, stream)
                       : launch_commit_t<float, bf16_t, false>(a, stream);
    case 2: return kda ? launch_commit_t<bf16_t, float, true>(a, stream)
                       : launch_commit_t<bf16_t, float, false>(a, stream);
    default: return kda ? launch_commit_t<bf16_t, bf16_t, true>(a, stream)
                        : launch_commit_t<bf16_t, bf16_t, false>(a, stream);
    }
}

hipError_t launch_conv_scatter(const ScatterArgs &a, hipStream_t stream)
{
    const int64_t units = (int64_t)3 * a.C * (a.conv_dtype ? 2 : 4) / 16;
    const unsigned gx = (unsigned)((units + 255) / 256);
    hipLaunchKernelGGL(conv_scatter_kernel, dim3(gx, (unsigned)a.B), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_track_copy(const TrackArgs &a, hipStream_t stream)
{
    const int64_t units = (a.ssm_row_b + a.conv_row_b) / 16;
    const int64_t blocks = (units + 255) / 256;
    const unsigned gx = (unsigned)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(track_copy_kernel, dim3(gx, (unsigned)a.B), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace la
