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
// values verify used.
//
// Verify has two forms.  Up to eight steps (the usual draft length) the chunk
// form: the steps' outputs and d come from one matrix-core product of the
// checkpoint with the steps' decayed keys and queries plus an 8x8 triangular
// recurrence, so the state is read once and no per-element arithmetic is
// spent on it.  Beyond eight steps the sequential form: one workgroup per
// (request, value head), the head's state rows spread over the waves as in
// the decode kernel (16-byte lane chunks, LPR lanes per row), held in fp32
// registers across the steps, every step running the per-row update the
// commit runs (the two agree bit for bit with an fp32 state).  It forms a
// chunk's q|k|v conv outputs, decays, norms and ring records up front, so
// its steps only update the state rows, with no barrier between steps.
// Commit stages the ring records of up to eight steps in LDS, with every
// load issued back to back, so a step waits for memory once per eight steps.
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

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
// The per-chunk front half of the sequential verify.  For the steps
// t0 .. t0 + nc - 1 of request b, value head h it
//   - stages the pre-conv inputs of the head's q|k|v channels in xe rows
//     3 .. 3 + nc - 1 below the three inputs before the chunk (rows 0 .. 2:
//     the conv state for the first chunk, else the previous chunk's last
//     three inputs), the gates in gs and the betas in bs;
//   - runs the short conv into ys (rounded to the I/O dtype, as a separate
//     conv kernel's output tensor would be), every (channel, step) from the
//     staged rows alone, so the work splits evenly over the threads;
//   - writes the conv windows (the history after each step: xe rows
//     tt + 1 .. tt + 3) and the ring records (rawk, rawv, g, beta and the
//     normalised k) with 16-byte stores where the rows allow;
//   - leaves the inverse norms in nq / nk and the decays exp(g) in gs.
// Ends with a barrier after everything later phases read from LDS.
constexpr int XLD = 3 * HD + 4;   // xe / ys row stride (floats): rows shift banks
constexpr int GLD = HD + 4;       // gs row stride (floats)

// 16 bytes of elements of type T from floats (nearest even for bf16).
template <typename T> struct V16;
template <> struct V16<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ uint4 pack(const float *v)
    {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3]));
    }
};
template <> struct V16<bf16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ uint4 pack(const float *v)
    {
        return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};
template <typename T>
__device__ __forceinline__ void store16(void *base, int64_t elem, const float *v)
{
    st_stream(static_cast<T *>(base) + elem, V16<T>::pack(v));
}

template <typename IOT, typename CT, bool KDA, bool CONV, int NT>
__device__ __forceinline__ void verify_front(const VerifyArgs &a, int b, int h, int kh, int slot,
                                             int rb, int t0, int nc, float (*xe)[XLD],
                                             float (*ys)[XLD], float (*gs)[GLD], float *bs,
                                             float *nq, float *nk)
{
    constexpr int NCH = 3 * HD;                                // q, k, v channels
    constexpr int XPT = (kChunk * NCH + NT - 1) / NT;          // staged inputs per thread
    constexpr int GPT = (kChunk * HD + NT - 1) / NT;           // staged gates per thread
    constexpr int HPT = (3 * NCH + NT - 1) / NT;               // history values per thread
    constexpr int IPT = (2 * NCH + NT - 1) / NT;               // conv items per thread
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RingArgs &R = a.ring;
    // The local channel j (over [q | k | v] of this head) -> global channel.
    auto glob = [&](int j) {
        return j < HD ? kh * HD + j
             : j < 2 * HD ? a.Hqk * HD + kh * HD + (j - HD) : 2 * a.Hqk * HD + h * HD + (j - 2 * HD);
    };
    // Conv items: item i = tid + NT m is channel i % NCH over the steps of
    // half i / NCH of the chunk (steps 4 half .. 4 half + 3).
    // ---- staging: every load issued back to back (indices clamped into the
    //      chunk, so no branch around a load).  The staging indices are
    //      re-derived from an opaque copy of the thread id in each chunk, so
    //      they are not kept live across chunks.
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    float4 wc[IPT];
    float bias[IPT];
    {
        float xv[XPT], gv2[GPT], hv[HPT], bv = 0.f;
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
            for (int m = 0; m < IPT; ++m) {
                const int gc = glob(min(ltid + NT * m, 2 * NCH - 1) % NCH);
                wc[m] = reinterpret_cast<const float4 *>(a.w)[gc];
                bias[m] = a.bias ? a.bias[gc] : 0.f;
            }
            if (t0 == 0) {  // the conv state: rows 0 .. 2
#pragma unroll
                for (int q = 0; q < HPT; ++q) {
                    const int i = min(ltid + q * NT, 3 * NCH - 1);
                    hv[q] = ld<CT>(a.conv_pool, (int64_t)slot * a.conv_stride +
                                                    (int64_t)(i / NCH) * a.C + glob(i % NCH));
                }
            } else {        // the previous (full) chunk's last three inputs
#pragma unroll
                for (int q = 0; q < HPT; ++q) {
                    const int i = min(tid + q * NT, 3 * NCH - 1);
                    hv[q] = round_to<CT>(xe[kChunk + i / NCH][i % NCH]);
                }
            }
        }
        __syncthreads();  // the previous chunk's staged values are no longer read
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int i = tid + q * NT;
            if (i < kChunk * NCH) xe[3 + i / NCH][i % NCH] = xv[q];
        }
        if constexpr (CONV) {
#pragma unroll
            for (int q = 0; q < HPT; ++q) {
                const int i = tid + q * NT;
                if (i < 3 * NCH) xe[i / NCH][i % NCH] = hv[q];
            }
        }
#pragma unroll
        for (int q = 0; q < GPT; ++q) {
            const int i = tid + q * NT;
            if (i < kChunk * HD) gs[i / HD][i % HD] = gv2[q];
        }
        if (tid < kChunk) bs[tid] = bv;
        __syncthreads();
    }
    // ---- the conv outputs, rounded to the I/O dtype
#pragma unroll
    for (int m = 0; m < IPT; ++m) {
        const int i = ltid + NT * m;
        if (i >= 2 * NCH) continue;
        const int j = i % NCH, t_lo = 4 * (i / NCH), t_hi = min(t_lo + 4, nc);
        if constexpr (CONV) {
            // taps: the history rounded to the conv dtype, the input as is
            float x0 = round_to<CT>(xe[t_lo][j]), x1 = round_to<CT>(xe[t_lo + 1][j]);
            float x2 = round_to<CT>(xe[t_lo + 2][j]);
            for (int tt = t_lo; tt < t_hi; ++tt) {
                const float x3 = xe[tt + 3][j];
                float acc = bias[m];
                acc = fmaf(wc[m].x, x0, acc);
                acc = fmaf(wc[m].y, x1, acc);
                acc = fmaf(wc[m].z, x2, acc);
                acc = fmaf(wc[m].w, x3, acc);
                ys[tt][j] = round_to<IOT>(silu(acc));
                x0 = x1;
                x1 = x2;
                x2 = round_to<CT>(x3);
            }
        } else {
            for (int tt = t_lo; tt < t_hi; ++tt) ys[tt][j] = xe[tt + 3][j];
        }
    }
    // ---- gates to the ring; then exp(g) per step
    for (int i = tid; i < nc * HD; i += NT) {
        const int tt = i / HD, c = i % HD;
        const int pos = (rb + t0 + tt) & (R.L - 1);
        const float g = gs[tt][c];
        if constexpr (KDA) R.g[ring_at(slot, a.Hv, R.L, h, pos, HD) + c] = g;
        else if (c == 0) R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)] = g;
        if (c == 0) R.beta[ring_at(slot, a.Hv, R.L, h, pos, 1)] = bs[tt];
        gs[tt][c] = fast_exp(g);
    }
    // ---- the conv windows: after step tt the history is xe rows
    //      tt + 1 .. tt + 3; q/k windows come from the first value head of
    //      the group only
    if constexpr (CONV) {
        constexpr int VN = V16<CT>::N, GR = HD / VN;  // channels per store, stores per block
        const int nblk = h % a.G == 0 ? 3 : 1, blk0 = 3 - nblk;
        for (int i = tid; i < nc * 3 * nblk * GR; i += NT) {
            const int grp = i % GR, blk = blk0 + (i / GR) % nblk, rr = (i / (GR * nblk)) % 3;
            const int tt = i / (GR * nblk * 3);
            const int j = blk * HD + grp * VN;
            float v[VN];
#pragma unroll
            for (int e = 0; e < VN; e += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(&xe[tt + 1 + rr][j + e]);
                v[e] = round_to<CT>(f.x); v[e + 1] = round_to<CT>(f.y);
                v[e + 2] = round_to<CT>(f.z); v[e + 3] = round_to<CT>(f.w);
            }
            store16<CT>(a.windows, (((int64_t)b * a.D + t0 + tt) * 3 + rr) * a.C + glob(j), v);
        }
    }
    __syncthreads();  // ys, gs complete
    // ---- the steps' norms, wave w taking steps w, w + NW, ..
    for (int tt = wave; tt < nc; tt += NW) {
        const float inv_q = inv_norm128(ys[tt][lane], ys[tt][lane + 64], a.eps);
        const float inv_k = inv_norm128(ys[tt][HD + lane], ys[tt][HD + lane + 64], a.eps);
        if (lane == 0) {
            nq[tt] = inv_q;
            nk[tt] = inv_k;
        }
    }
    __syncthreads();  // nq, nk complete
    // ---- ring vectors rawk, rawv and the normalised k, 16 bytes a store
    {
        constexpr int VN = V16<IOT>::N, GR = HD / VN;
        for (int i = tid; i < nc * 3 * GR; i += NT) {
            const int grp = i % GR, which = (i / GR) % 3, tt = i / (3 * GR);
            const int pos = (rb + t0 + tt) & (R.L - 1);
            const int c = grp * VN, src = which == 1 ? 2 * HD + c : HD + c;
            const float sc = which == 2 ? nk[tt] : 1.f;
            float v[VN];
#pragma unroll
            for (int e = 0; e < VN; e += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(&ys[tt][src + e]);
                v[e] = f.x * sc; v[e + 1] = f.y * sc; v[e + 2] = f.z * sc; v[e + 3] = f.w * sc;
            }
            void *dst = which == 0 ? R.rawk : which == 1 ? R.rawv : R.k;
            store16<IOT>(dst, ring_at(slot, a.Hv, R.L, h, pos, HD) + c, v);
        }
    }
}

// Sequential form, any number of steps: the state rows are carried in fp32
// registers and every step runs the per-row update the commit runs.
template <typename ST, typename IOT, typename CT, bool KDA, bool CONV>
__global__ void __launch_bounds__((DecodeCfg<HD, ST>::NT)) verify_kernel(VerifyArgs a)
{
    using Cfg = DecodeCfg<HD, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = Cfg::NT;
    __shared__ __align__(16) float xe[kChunk + 3][XLD];  // the chunk's inputs below the three before it
    __shared__ __align__(16) float ys[kChunk][XLD];      // the chunk's q|k|v (conv outputs)
    __shared__ float gs[kChunk][GLD];          // the chunk's decays exp(g) (GDN: broadcast)
    __shared__ float nq[kChunk], nk[kChunk];   // the chunk's inverse q and k norms
    __shared__ float bs[kChunk];               // the chunk's betas

    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv, kh = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = a.slots[b], rb = a.ring_base[b];
    const int n = min(max(a.n_tok[b], 0), a.D);
    auto out_at = [&](int t, int i) { return (((int64_t)b * a.D + t) * a.Hv + h) * HD + i; };
    const int first_zero = (slot < 0 || slot >= a.num_rows) ? 0 : n;
    for (int i = tid + first_zero * HD; i < a.D * HD; i += NT)  // steps past n (or a skipped entry)
        st<IOT>(a.out, out_at(i / HD, i % HD), 0.f);
    if (first_zero == 0) return;

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
        const int nc = min(kChunk, n - t0);
        verify_front<IOT, CT, KDA, CONV, NT>(a, b, h, kh, slot, rb, t0, nc, xe, ys, gs, bs, nq, nk);
        // ---- the steps: only the state rows, with no barrier between steps
        for (int tt = 0; tt < nc; ++tt) {
            const int t = t0 + tt;
            const int pos = (rb + t) & (R.L - 1);
            const float inv_q = nq[tt], inv_k = nk[tt];
            float kk[EPL], qq[EPL], al[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kk[e] = ys[tt][HD + col0 + e] * inv_k;
                qq[e] = ys[tt][col0 + e] * inv_q;
                al[e] = gs[tt][col0 + e];
            }
            const float beta = bs[tt];
            // every lane of a row group gets the row's sums; lane (l % LPR == j)
            // keeps row instruction j's, so each lane stores once per step
            float my_o = 0.f, my_d = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = (wave * NJ + j) * RPW + lane / LPR;
                const float d = row_step<EPL, LPR>(s[j], al, kk, ys[tt][2 * HD + r], beta);
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

// Chunk form, at most kChunk steps (one chunk).  With G_t the running sum of
// the log-decays over the steps (per channel; GDN: per head), k_t, q_t the
// normalised keys and queries and S the checkpoint, the state the sequential
// rule holds after its decay at step t is
//   S'_t = S Diag(e^{G_t}) + sum_{j<t} d_j (k_j * e^{G_t - G_j})^T,
// so with X = S [K~ | Q~]  (K~_t = k_t * e^{G_t}, Q~_t = q_t * e^{G_t}),
//   A_tj = sum_c k_t[c] k_j[c] e^{G_t[c] - G_j[c]}   (j < t),
//   P_tj = sum_c q_t[c] k_j[c] e^{G_t[c] - G_j[c]}   (j <= t):
//   d_t = beta_t (v_t - X[:, t] - sum_{j<t} A_tj d_j),
//   o_t = scale (X[:, 8 + t] + sum_{j<=t} P_tj d_j).
// Every exponent is <= 0.  The one product that touches the state, X, is a
// 128 x 16 x 128 matrix-core product per head (bf16 state: the state is the
// exact bf16 operand and [K~ | Q~] a two-term bf16 split; fp32 state:
// v_mfma_f32_16x16x4f32), so the state crosses HBM once and no per-element
// arithmetic is spent on it.
//
// Phases (three workgroup barriers; records and outputs are written with
// non-temporal stores):
//   1. staging: 16-byte loads of the head's inputs, conv state, conv weights
//      and gates; the gates' running sums and their ring records by 32 lanes
//      holding four channels each;
//   2. the state fragments are issued (they stream in under this phase);
//      one step per wave: the conv of the step's q, k and v channels (two
//      of each per lane), the q and k norms (wave sums), the ring records,
//      the conv window and the step's rows of [K~ | Q~];
//   3. the matrix-core product (every wave) and A, P (eight lanes per pair);
//   4. the d recurrence and the outputs per value row.
template <typename T> __device__ __forceinline__ void store2(void *base, int64_t elem, float v0, float v1);
template <> __device__ __forceinline__ void store2<float>(void *base, int64_t elem, float v0, float v1)
{
    float *p = static_cast<float *>(base) + elem;
    __builtin_nontemporal_store(v0, p);
    __builtin_nontemporal_store(v1, p + 1);
}
template <> __device__ __forceinline__ void store2<bf16_t>(void *base, int64_t elem, float v0, float v1)
{
    __builtin_nontemporal_store(pack_bf16x2(v0, v1), reinterpret_cast<uint32_t *>(static_cast<bf16_t *>(base) + elem));
}
// 16 bytes of T as floats.
template <typename T> __device__ __forceinline__ void unpack16(const uint4 &r, float *v);
template <> __device__ __forceinline__ void unpack16<float>(const uint4 &r, float *v)
{
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
    v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
}
template <> __device__ __forceinline__ void unpack16<bf16_t>(const uint4 &r, float *v)
{
    Stor<bf16_t>::unpack(r, v);
}

constexpr int kChunkNT = 512;   // threads of the chunk-form verify workgroup

// Floor of a log decay inside the running sums of the chunk forms and the
// fold.  They use differences G_t - G_j of running sums, which a gate of -inf (a full
// reset of the state) would turn into -inf - -inf.  exp(-128) is below the
// smallest fp32 denormal, so a single step's decay is already exactly 0 at the
// floor: the floor changes no result, while every running sum stays finite.
constexpr float kGFloor = -128.f;

template <typename ST, typename IOT, typename CT, bool KDA, bool CONV>
__global__ void __launch_bounds__(kChunkNT) verify_chunk_kernel(VerifyArgs a)
{
    constexpr int NT = kChunkNT, NW = NT / 64;
    constexpr int TPW = HD / 16 / NW;               // 16-row state tiles per wave
    constexpr int LPP = NT >= 512 ? 8 : 4;          // lanes per (t, j) pair of A and P
    static_assert(TPW * NW * 16 == HD && HD <= NT, "layout");
    constexpr int LDB = HD + 4;                     // [K~ | Q~] row stride (floats)
    constexpr int LDBH = HD + 8;                    // its bf16 hi / lo row stride (elements)
    constexpr bool kBf16B = sizeof(ST) == 2;        // [K~ | Q~] kept as bf16 hi + lo
    constexpr int BSZ = kBf16B ? 16 * LDBH : 16 * LDB;  // floats
    // taps from the inputs need rounding to the conv dtype only when it is
    // narrower than the I/O dtype
    constexpr bool kRoundTaps = std::is_same<CT, bf16_t>::value && !std::is_same<IOT, CT>::value;
    constexpr int LDX = 17;                         // X row stride (floats)
    constexpr int FR = HD * (int)sizeof(ST) / 64;   // 64-byte row pieces: 4 (bf16) or 8 (fp32)
    constexpr int NCH = 3 * HD;
    __shared__ __align__(16) float xe[kChunk + 3][XLD];  // conv state rows 0..2, inputs below
    __shared__ __align__(16) float ys[kChunk][XLD];      // q|k|v conv outputs
    __shared__ __align__(16) float Gs[kChunk][GLD];      // running sums of the log-decays
    // [K~ | Q~]: rows t: K~_t, rows 8 + t: Q~_t; fp32 (fp32 state) or the
    // bf16 hi rows followed by the bf16 lo rows (bf16 state)
    __shared__ __align__(16) float Braw[BSZ];
    float (*Bm)[LDB] = reinterpret_cast<float (*)[LDB]>(Braw);
    bf16_t (*Bh)[LDBH] = reinterpret_cast<bf16_t (*)[LDBH]>(Braw);
    bf16_t (*Bl)[LDBH] = Bh + 16;
    // X = S [K~ | Q~]^T after the product; the conv weights and biases before
    __shared__ __align__(16) float Xw[HD * LDX > 5 * NCH ? HD * LDX : 5 * NCH];
    __shared__ float Am[kChunk][kChunk], Pm[kChunk][kChunk];
    __shared__ float nq[kChunk], nk[kChunk], bs[kChunk];
    float4 *w4 = reinterpret_cast<float4 *>(Xw);     // [NCH] conv weights
    float *wb = Xw + 4 * NCH;                         // [NCH] conv biases

    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv, kh = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int slot = a.slots[b], rb = a.ring_base[b];
    const int n = min(max(a.n_tok[b], 0), a.D);
    auto out_at = [&](int t, int i) { return (((int64_t)b * a.D + t) * a.Hv + h) * HD + i; };
    const int first_zero = (slot < 0 || slot >= a.num_rows) ? 0 : n;
    for (int i = tid + first_zero * HD; i < a.D * HD; i += NT)  // steps past n (or a skipped entry)
        st<IOT>(a.out, out_at(i / HD, i % HD), 0.f);
    if (first_zero == 0) return;

    const RingArgs &R = a.ring;
    // first global channel of block blk (0 = q, 1 = k, 2 = v) of this head
    auto gbase = [&](int blk) {
        return blk == 0 ? kh * HD : blk == 1 ? (a.Hqk + kh) * HD : 2 * a.Hqk * HD + h * HD;
    };
    auto pos_of = [&](int t) { return (rb + t) & (R.L - 1); };

    // ---- 1. staging ------------------------------------------------------
    constexpr int VX = V16<IOT>::N, GX = HD / VX, NX = kChunk * 3 * GX, XI = (NX + NT - 1) / NT;
    constexpr int VH = V16<CT>::N, GH = HD / VH, NH = 3 * 3 * GH, HI = (NH + NT - 1) / NT;
    static_assert(NCH <= 2 * NT, "two conv weight vectors per thread");
    uint4 xr[XI], hr[HI];
    float4 g4[kChunk], wr0, wr1 = make_float4(0.f, 0.f, 0.f, 0.f), br = make_float4(0.f, 0.f, 0.f, 0.f);
    float bv = 0.f;
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int i = min(tid + q * NT, NX - 1), grp = i % GX, blk = (i / GX) % 3;
        const int tt = min(i / (3 * GX), n - 1);
        xr[q] = *reinterpret_cast<const uint4 *>(static_cast<const IOT *>(a.x) +
                                                 ((int64_t)b * a.D + tt) * a.C + gbase(blk) + grp * VX);
    }
    if (tid < 32) {  // lane l: channels 4 l .. 4 l + 3 of every step
#pragma unroll
        for (int tt = 0; tt < kChunk; ++tt) {
            const int64_t bt = (int64_t)b * a.D + min(tt, n - 1);
            if constexpr (KDA) {
                g4[tt] = *reinterpret_cast<const float4 *>(a.g + (bt * a.Hv + h) * HD + 4 * tid);
            } else {
                const float g1 = a.g[bt * a.Hv + h];
                g4[tt] = make_float4(g1, g1, g1, g1);
            }
        }
    }
    if (tid < kChunk) bv = a.beta[((int64_t)b * a.D + min(tid, n - 1)) * a.Hv + h];
    if constexpr (CONV) {
#pragma unroll
        for (int q = 0; q < HI; ++q) {
            const int i = min(tid + q * NT, NH - 1), grp = i % GH, blk = (i / GH) % 3, r = i / (3 * GH);
            hr[q] = *reinterpret_cast<const uint4 *>(static_cast<const CT *>(a.conv_pool) +
                                                     (int64_t)slot * a.conv_stride + (int64_t)r * a.C +
                                                     gbase(blk) + grp * VH);
        }
        {
            const int j0 = min(tid, NCH - 1), j1 = min(tid + NT, NCH - 1);
            wr0 = reinterpret_cast<const float4 *>(a.w)[gbase(j0 / HD) + j0 % HD];
            if constexpr (NT < NCH) wr1 = reinterpret_cast<const float4 *>(a.w)[gbase(j1 / HD) + j1 % HD];
        }
        if (tid < NCH / 4 && a.bias)
            br = *reinterpret_cast<const float4 *>(a.bias + gbase(tid / (HD / 4)) + 4 * (tid % (HD / 4)));
    }

#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int i = tid + q * NT, grp = i % GX, blk = (i / GX) % 3, tt = i / (3 * GX);
        if (i < NX && tt < n) {
            float v[VX];
            unpack16<IOT>(xr[q], v);
#pragma unroll
            for (int e = 0; e < VX; e += 4)
                *reinterpret_cast<float4 *>(&xe[3 + tt][blk * HD + grp * VX + e]) =
                    make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
        }
    }
    if constexpr (CONV) {
#pragma unroll
        for (int q = 0; q < HI; ++q) {
            const int i = tid + q * NT, grp = i % GH, blk = (i / GH) % 3, r = i / (3 * GH);
            if (i < NH) {
                float v[VH];
                unpack16<CT>(hr[q], v);
#pragma unroll
                for (int e = 0; e < VH; e += 4)
                    *reinterpret_cast<float4 *>(&xe[r][blk * HD + grp * VH + e]) =
                        make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
            }
        }
        if (tid < NCH) w4[tid] = wr0;
        if (tid + NT < NCH) w4[tid + NT] = wr1;
        if (tid < NCH / 4) *reinterpret_cast<float4 *>(&wb[4 * tid]) = br;
    }
    if (tid < kChunk) {
        bs[tid] = bv;
        if (tid < n) R.beta[ring_at(slot, a.Hv, R.L, h, pos_of(tid), 1)] = bv;
    }
    if (tid < 32) {
        float4 G = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int tt = 0; tt < kChunk; ++tt) {
            if (tt < n) {
                if constexpr (KDA)
                    *reinterpret_cast<float4 *>(R.g + ring_at(slot, a.Hv, R.L, h, pos_of(tt), HD) + 4 * tid) = g4[tt];
                else if (tid == 0)
                    R.g[ring_at(slot, a.Hv, R.L, h, pos_of(tt), 1)] = g4[tt].x;
                G.x += fmaxf(g4[tt].x, kGFloor); G.y += fmaxf(g4[tt].y, kGFloor);
                G.z += fmaxf(g4[tt].z, kGFloor); G.w += fmaxf(g4[tt].w, kGFloor);
                *reinterpret_cast<float4 *>(&Gs[tt][4 * tid]) = G;
            }
        }
    }
    for (int i = tid; i < 16 * (HD / 4); i += NT) {  // rows of [K~ | Q~] past n are zero
        const int r = i / (HD / 4), c = 4 * (i % (HD / 4));
        if ((r & (kChunk - 1)) >= n) {
            if constexpr (kBf16B) {
                *reinterpret_cast<uint2 *>(&Bh[r][c]) = make_uint2(0, 0);
                *reinterpret_cast<uint2 *>(&Bl[r][c]) = make_uint2(0, 0);
            } else {
                *reinterpret_cast<float4 *>(&Bm[r][c]) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    __syncthreads();

    // The state as matrix-core operand fragments, issued after the staged
    // inputs have landed, so they stream in while the units below run: wave
    // w owns the TPW 16-row tiles from row 16 TPW w; lane (li, lq) holds 16
    // bytes at byte 64 f + 16 lq of row li of a tile.  bf16: fragment f is
    // k = 32 f + 8 lq + e (e < 8), one 16x16x32 step; fp32: fragment f is
    // k = 16 f + 4 lq + e (e < 4), four 16x16x4 steps.
    __builtin_amdgcn_sched_barrier(0);
    const char *S = static_cast<const char *>(a.ssm_pool) +
                    ((int64_t)slot * a.ssm_stride + (int64_t)h * HD * HD) * sizeof(ST);
    uint4 fr[TPW][FR];
#pragma unroll
    for (int T = 0; T < TPW; ++T)
#pragma unroll
        for (int f = 0; f < FR; ++f)
            fr[T][f] = ld_stream(S + (int64_t)(16 * (TPW * wave + T) + li) * HD * sizeof(ST) + 64 * f + 16 * lq);
    __builtin_amdgcn_sched_barrier(0);
    // ---- 2. one step per wave: the conv of the step's q, k and v channels
    //      (two of each block per lane), norms, records and window
    const bool qk_win = h % a.G == 0;  // q/k windows come from the group's first head
    for (int tt = wave; tt < n; tt += NW) {
        const int64_t rr = ring_at(slot, a.Hv, R.L, h, pos_of(tt), HD) + 2 * lane;
        const int64_t wrow = ((int64_t)b * a.D + tt) * 3 * a.C + 2 * lane;
        float yq0 = 0.f, yq1 = 0.f, yk0 = 0.f, yk1 = 0.f;
#pragma unroll
        for (int blk = 0; blk < 3; ++blk) {
            const int j = blk * HD + 2 * lane;
            const float2 r3 = *reinterpret_cast<const float2 *>(&xe[tt + 3][j]);
            float y0 = r3.x, y1 = r3.y;
            if constexpr (CONV) {
                const float2 r0 = *reinterpret_cast<const float2 *>(&xe[tt][j]);
                const float2 r1 = *reinterpret_cast<const float2 *>(&xe[tt + 1][j]);
                const float2 r2 = *reinterpret_cast<const float2 *>(&xe[tt + 2][j]);
                const float4 wa = w4[j], wc = w4[j + 1];
                const float2 bb = *reinterpret_cast<const float2 *>(&wb[j]);
                auto tap = [](float x) { return kRoundTaps ? round_to<CT>(x) : x; };
                float acc0 = bb.x, acc1 = bb.y;
                acc0 = fmaf(wa.x, tap(r0.x), acc0);
                acc0 = fmaf(wa.y, tap(r1.x), acc0);
                acc0 = fmaf(wa.z, tap(r2.x), acc0);
                acc0 = fmaf(wa.w, r3.x, acc0);
                acc1 = fmaf(wc.x, tap(r0.y), acc1);
                acc1 = fmaf(wc.y, tap(r1.y), acc1);
                acc1 = fmaf(wc.z, tap(r2.y), acc1);
                acc1 = fmaf(wc.w, r3.y, acc1);
                y0 = round_to<IOT>(silu(acc0));
                y1 = round_to<IOT>(silu(acc1));
                // the history after step tt (the store rounds to the conv dtype)
                if (blk == 2 || qk_win) {
                    const int64_t w0 = wrow + gbase(blk);
                    store2<CT>(a.windows, w0, r1.x, r1.y);
                    store2<CT>(a.windows, w0 + a.C, r2.x, r2.y);
                    store2<CT>(a.windows, w0 + 2 * a.C, r3.x, r3.y);
                }
            }
            *reinterpret_cast<float2 *>(&ys[tt][j]) = make_float2(y0, y1);
            if (blk == 0) { yq0 = y0; yq1 = y1; }
            if (blk == 1) { yk0 = y0; yk1 = y1; store2<IOT>(R.rawk, rr, y0, y1); }
            if (blk == 2) store2<IOT>(R.rawv, rr, y0, y1);
            __builtin_amdgcn_sched_barrier(0);  // one block's operands live at a time
        }
        const float iq = __builtin_amdgcn_rsqf(wave_sum(fmaf(yq1, yq1, yq0 * yq0)) + a.eps);
        const float ik = __builtin_amdgcn_rsqf(wave_sum(fmaf(yk1, yk1, yk0 * yk0)) + a.eps);
        if (lane == 0) {
            nq[tt] = iq;
            nk[tt] = ik;
        }
        store2<IOT>(R.k, rr, yk0 * ik, yk1 * ik);
        const float2 G = *reinterpret_cast<const float2 *>(&Gs[tt][2 * lane]);
        const float e0 = fast_exp(G.x), e1 = fast_exp(G.y);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const float b0 = (blk ? yk0 * ik : yq0 * iq) * e0, b1 = (blk ? yk1 * ik : yq1 * iq) * e1;
            const int row = blk == 1 ? tt : kChunk + tt;
            if constexpr (kBf16B) {  // the two-term split: hi = bf16(b), lo = bf16(b - hi)
                const uint32_t hp = pack_bf16x2(b0, b1);
                *reinterpret_cast<uint32_t *>(&Bh[row][2 * lane]) = hp;
                *reinterpret_cast<uint32_t *>(&Bl[row][2 * lane]) =
                    pack_bf16x2(b0 - bf16_lo(hp), b1 - bf16_hi(hp));
            } else {
                *reinterpret_cast<float2 *>(&Bm[row][2 * lane]) = make_float2(b0, b1);
            }
        }
    }
    __syncthreads();

    // ---- 3. X = S [K~ | Q~]^T on the matrix cores (lane (li, lq) ends with
    //      X[16 (TPW w + T) + 4 lq + r][li] in acc[T][r]), and A, P
    f32x4 acc[TPW];
#pragma unroll
    for (int T = 0; T < TPW; ++T) acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(ST) == 2) {
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&Bh[li][32 * f + 8 * lq]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&Bl[li][32 * f + 8 * lq]);
#pragma unroll
            for (int T = 0; T < TPW; ++T) {
                const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fr[T][f]);
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[T], 0, 0, 0);
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[T], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const float4 bq = *reinterpret_cast<const float4 *>(&Bm[li][16 * f + 4 * lq]);
            const float bv4[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int T = 0; T < TPW; ++T) {
                    const uint32_t w = e == 0 ? fr[T][f].x : e == 1 ? fr[T][f].y : e == 2 ? fr[T][f].z : fr[T][f].w;
                    acc[T] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w), bv4[e], acc[T], 0, 0, 0);
                }
        }
    }
    float (*Xs)[LDX] = reinterpret_cast<float (*)[LDX]>(Xw);  // the weights are no longer read
#pragma unroll
    for (int T = 0; T < TPW; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) Xs[16 * (TPW * wave + T) + 4 * lq + r][li] = acc[T][r];
    // A and P: pair p of the 36 pairs (t, j <= t) on the LPP aligned lanes
    // from thread NT - 36 LPP + LPP p, which split the channels
    if (tid >= NT - LPP * 36) {
        const int p = (tid - (NT - LPP * 36)) / LPP, qc = tid % LPP;
        int t = 0;
        while ((t + 1) * (t + 2) / 2 <= p) ++t;
        const int j = p - t * (t + 1) / 2;
        float sa = 0.f, sp = 0.f;
        if (t < n) {
            for (int m = 0; m < HD / LPP; ++m) {
                const int c = qc + LPP * m;
                const float w = ys[j][HD + c] * fast_exp(Gs[t][c] - Gs[j][c]);
                sa = fmaf(ys[t][HD + c], w, sa);
                sp = fmaf(ys[t][c], w, sp);
            }
        }
        sa = group_sum<LPP>(sa);
        sp = group_sum<LPP>(sp);
        if (qc == 0 && t < n) {
            Am[t][j] = j < t ? sa * nk[t] * nk[j] : 0.f;
            Pm[t][j] = sp * nq[t] * nk[j];
        }
    }
    __syncthreads();

    // ---- 4. per value row r: the d recurrence, then the outputs
    if (tid < HD) {
        const int r = tid;
        float d[kChunk];
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            d[t] = 0.f;
            if (t < n) {
                float u = Xs[r][t];
#pragma unroll
                for (int jj = 0; jj < t; ++jj) u = fmaf(Am[t][jj], d[jj], u);
                d[t] = bs[t] * (ys[t][2 * HD + r] - u);
            }
        }
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            if (t < n) {
                float o = Xs[r][kChunk + t];
#pragma unroll
                for (int jj = 0; jj <= t; ++jj) o = fmaf(Pm[t][jj], d[jj], o);
                st<IOT>(a.out, out_at(t, r), a.scale * o);
                st<IOT>(R.d, ring_at(slot, a.Hv, R.L, h, pos_of(t), HD) + r, d[t]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// commit
// ---------------------------------------------------------------------------
// One 512-thread workgroup per (request, value head).  Up to eight accepted
// steps take the chunk form below; more take the sequential replay, whose
// per-row arithmetic is the sequential verify's (bit for bit with an fp32
// state).
constexpr int kCommitNT = 512;

// Rows of a head spread over NW waves as in the decode kernel: LPR lanes of
// EPL elements (16 bytes) per row, NJ row instructions per lane.
template <typename ST, int NW_> struct RowCfg {
    static constexpr int NW = NW_;
    static constexpr int EPL = Stor<ST>::kPer16B, LPR = HD / EPL, RPW = 64 / LPR;
    static constexpr int NJ = HD / RPW / NW;
    static_assert(NJ * RPW * NW == HD, "rows split evenly over the waves");
};

// The sequential replay of na (> 0) ring steps onto the state row.
template <typename ST, typename IOT, bool KDA>
__device__ __forceinline__ void commit_sequential(const CommitArgs &a, int b, int h, int slot, int na,
                                                  float (*ks)[HD], float (*vs)[HD], float (*gsh)[HD],
                                                  float *bsh, float *nk)
{
    using Cfg = RowCfg<ST, kCommitNT / 64>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = kCommitNT;
    constexpr int VPT = (kChunk * HD + NT - 1) / NT;  // staged ring values per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = a.ring_base[b];
    ST *S = static_cast<ST *>(a.ssm_pool) + (int64_t)slot * a.ssm_stride + (int64_t)h * HD * HD;
    const int col0 = (lane % LPR) * EPL;
    auto row_of = [&](int j) { return (wave * NJ + j) * RPW + lane / LPR; };
    float s[NJ][EPL];
#pragma unroll
    for (int j = 0; j < NJ; ++j) Stor<ST>::unpack(ld_stream(S + (int64_t)row_of(j) * HD + col0), s[j]);
    const RingArgs &R = a.ring;
    for (int t0 = 0; t0 < na; t0 += kChunk) {
        // stage the chunk's ring records in LDS, all loads back to back
        const int nc = min(kChunk, na - t0);
        float kv[VPT], vv[VPT], gv[VPT], bv = 0.f;
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int i = min(tid + q * NT, kChunk * HD - 1);
            const int pos = (rb + t0 + min(i / HD, nc - 1)) & (R.L - 1);
            const int64_t vr = ring_at(slot, a.Hv, R.L, h, pos, HD) + i % HD;
            kv[q] = ld<IOT>(R.rawk, vr);
            vv[q] = ld<IOT>(R.rawv, vr);
            gv[q] = KDA ? R.g[vr] : R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)];
        }
        if (tid < kChunk) bv = R.beta[ring_at(slot, a.Hv, R.L, h, (rb + t0 + min(tid, nc - 1)) & (R.L - 1), 1)];
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
            for (int j = 0; j < NJ; ++j) row_step<EPL, LPR>(s[j], al, kk, vs[tt][row_of(j)], beta);
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) st_stream(S + (int64_t)row_of(j) * HD + col0, Stor<ST>::pack(s[j]));
}

// Chunk form of the commit of na <= 8 steps.  With G_t the running sum of
// the steps' log-decays, k_t the normalised keys and S the checkpoint, d_t
// follows from X = S K~^T (K~_t = k_t * e^{G_t}) and the 8x8 A of the verify's
// chunk form, and the committed state is
//   S_na = S Diag(e^{G_na}) + sum_t d_t (k_t * e^{G_na - G_t})^T,
// the second term a rank-8 product on the matrix cores.  Wave w owns state
// rows 16 w .. 16 w + 15; lane (m, g) holds row 16 w + m, columns
// 32 c + 8 g .. 32 c + 8 g + 7 for c < 4, in fp32 after loading.
//   X:      bf16 state: v_mfma_f32_16x16x32_bf16, the state exact and K~ split
//           into bf16 hi + lo; fp32 state: v_mfma_f32_16x16x4f32 with lane
//           group g supplying column 32 c + 8 g + e for step (c, e);
//   A (the 28 pairs j < t) is formed beside the K~ / KD rows; after that
//   barrier each wave runs X, d and the update for its own rows alone.
//   update: for each column block c and half hf, D[i][m] = sum_t KD_t[col(i)]
//           d_t[row m] with col(i) = 32 c + 8 (i / 4) + 4 hf + i % 4, so lane
//           (m, g) receives columns 32 c + 8 g + 4 hf .. + 3 of its own row,
//           accumulated onto S e^{G_na} of the same elements.
template <typename ST, typename IOT, bool KDA>
__global__ void __launch_bounds__(kCommitNT) commit_kernel(CommitArgs a)
{
    constexpr int NT = kCommitNT;
    constexpr int LDB = HD + 4, LDBH = HD + 8, LDX = kChunk + 1;
    constexpr bool kBf16 = sizeof(ST) == 2;
    __shared__ __align__(16) float ks[kChunk][HD];   // rawk (the sequential form: the same)
    __shared__ __align__(16) float vs[kChunk][HD];   // rawv
    __shared__ __align__(16) float gsh[kChunk][HD];  // G_t (the sequential form: g, exp g)
    __shared__ float bsh[kChunk], nk[kChunk];
    __shared__ __align__(16) float Braw[kBf16 ? kChunk * LDBH : kChunk * LDB];  // K~
    __shared__ __align__(16) float KD[kChunk][LDB];  // k_t e^{G_na - G_t}
    __shared__ __align__(16) float Ds[kChunk][HD];   // d_t
    __shared__ float Xs[HD][LDX];
    __shared__ float Am[kChunk][kChunk];
    __shared__ __align__(16) float Ee[HD];           // e^{G_na}
    float (*Bm)[LDB] = reinterpret_cast<float (*)[LDB]>(Braw);
    bf16_t (*Bh)[LDBH] = reinterpret_cast<bf16_t (*)[LDBH]>(Braw);
    bf16_t (*Bl)[LDBH] = reinterpret_cast<bf16_t (*)[LDBH]>(Braw) + kChunk;

    const int b = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int slot = a.slots[b];
    const int na = min(a.accepted[b], a.ring.L);
    if (slot < 0 || slot >= a.num_rows || na <= 0) return;  // nothing accepted: row unchanged
    if (na > kChunk) {
        commit_sequential<ST, IOT, KDA>(a, b, h, slot, na, ks, vs, gsh, bsh, nk);
        return;
    }
    const RingArgs &R = a.ring;
    const int rb = a.ring_base[b];
    auto pos_of = [&](int t) { return (rb + t) & (R.L - 1); };

    // ---- 1. staging: rawk / rawv rows (16-byte loads), gates, betas
    constexpr int VI = V16<IOT>::N, GI = HD / VI, NI = kChunk * 2 * GI, II = (NI + NT - 1) / NT;
    uint4 xr[II];
    float gv[kChunk], bv = 0.f;
#pragma unroll
    for (int q = 0; q < II; ++q) {
        const int i = min(tid + q * NT, NI - 1), grp = i % GI, which = (i / GI) % 2;
        const int t = min(i / (2 * GI), na - 1);
        xr[q] = *reinterpret_cast<const uint4 *>(static_cast<const IOT *>(which ? R.rawv : R.rawk) +
                                                 ring_at(slot, a.Hv, R.L, h, pos_of(t), HD) + grp * VI);
    }
    if (tid < kChunk) bv = R.beta[ring_at(slot, a.Hv, R.L, h, pos_of(min(tid, na - 1)), 1)];
    if (tid < HD) {  // thread c: channel c of every step
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            const int pos = pos_of(min(t, na - 1));
            gv[t] = KDA ? R.g[ring_at(slot, a.Hv, R.L, h, pos, HD) + tid] : R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)];
        }
    }
    // The state, issued right behind the ring records: vector loads return
    // in order, so the staging below waits for its own data only and the
    // state streams in under phase 2.  Lane (m, g) of wave w: row 16 w + m,
    // columns 32 c + 8 g .. 32 c + 8 g + 7 for c < 4.
    const char *Sb = static_cast<const char *>(a.ssm_pool) +
                     ((int64_t)slot * a.ssm_stride + (int64_t)h * HD * HD) * sizeof(ST);
    const char *Srow = Sb + (int64_t)(16 * wave + m) * HD * sizeof(ST);
    constexpr int LPB = kBf16 ? 1 : 2;   // 16-byte loads per 8-column block
    uint4 fr[4][LPB];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int l = 0; l < LPB; ++l)
            fr[c][l] = ld_stream(Srow + (int64_t)(32 * c + 8 * g) * sizeof(ST) + 16 * l);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < II; ++q) {
        const int i = tid + q * NT, grp = i % GI, which = (i / GI) % 2, t = i / (2 * GI);
        if (i < NI && t < na) {
            float v[VI];
            unpack16<IOT>(xr[q], v);
            float *dst = which ? &vs[t][grp * VI] : &ks[t][grp * VI];
#pragma unroll
            for (int e = 0; e < VI; e += 4)
                *reinterpret_cast<float4 *>(dst + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
        }
    }
    if (tid < kChunk) bsh[tid] = bv;
    if (tid < HD) {
        float G = 0.f;
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            if (t < na) {
                G += fmaxf(gv[t], kGFloor);
                gsh[t][tid] = G;
            }
        }
        Ee[tid] = fast_exp(G);
    }
    for (int i = tid; i < kChunk * (HD / 4); i += NT) {  // rows past na are zero
        const int t = i / (HD / 4), c = 4 * (i % (HD / 4));
        if (t >= na) {
            *reinterpret_cast<float4 *>(&KD[t][c]) = make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4 *>(&Ds[t][c]) = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (kBf16) {
                *reinterpret_cast<uint2 *>(&Bh[t][c]) = make_uint2(0, 0);
                *reinterpret_cast<uint2 *>(&Bl[t][c]) = make_uint2(0, 0);
            } else {
                *reinterpret_cast<float4 *>(&Bm[t][c]) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    __syncthreads();

    // ---- 2. per step wave: the k norm, the row of K~ and the row of KD
    for (int t = wave; t < na; t += NT / 64) {
        const float2 kr = *reinterpret_cast<const float2 *>(&ks[t][2 * lane]);
        const float ik = __builtin_amdgcn_rsqf(wave_sum(fmaf(kr.y, kr.y, kr.x * kr.x)) + a.eps);
        if (lane == 0) nk[t] = ik;
        const float2 G = *reinterpret_cast<const float2 *>(&gsh[t][2 * lane]);
        const float k0 = kr.x * ik, k1 = kr.y * ik;
        const float b0 = k0 * fast_exp(G.x), b1 = k1 * fast_exp(G.y);
        if constexpr (kBf16) {  // the two-term split: hi = bf16(b), lo = bf16(b - hi)
            const uint32_t hp = pack_bf16x2(b0, b1);
            *reinterpret_cast<uint32_t *>(&Bh[t][2 * lane]) = hp;
            *reinterpret_cast<uint32_t *>(&Bl[t][2 * lane]) = pack_bf16x2(b0 - bf16_lo(hp), b1 - bf16_hi(hp));
        } else {
            *reinterpret_cast<float2 *>(&Bm[t][2 * lane]) = make_float2(b0, b1);
        }
        // e^{G_na - G_t} as a quotient of exponentials would overflow for
        // strong decays; formed directly it is <= 1
        const float2 Gn = *reinterpret_cast<const float2 *>(&gsh[na - 1][2 * lane]);
        *reinterpret_cast<float2 *>(&KD[t][2 * lane]) =
            make_float2(k0 * fast_exp(Gn.x - G.x), k1 * fast_exp(Gn.y - G.y));
    }
    // A_tj = k_t . k_j e^{G_t - G_j} (j < t): 28 pairs on eight lanes each
    if (tid >= NT - 8 * 28) {
        const int p = (tid - (NT - 8 * 28)) / 8, qc = tid % 8;
        int t = 1;
        while (t * (t + 1) / 2 <= p) ++t;
        const int j = p - t * (t - 1) / 2;
        float sa = 0.f;
        if (t < na) {
            for (int mm = 0; mm < HD / 8; ++mm) {
                const int c = qc + 8 * mm;
                sa = fmaf(ks[t][c], ks[j][c] * fast_exp(gsh[t][c] - gsh[j][c]), sa);
            }
        }
        sa = group_sum<8>(sa);
        if (qc == 0 && t < na) Am[t][j] = sa;  // unnormalised: scaled below
    }
    __syncthreads();
    // From here each wave works on its own 16 rows alone: its rows of X and
    // d go through LDS within the wave only, so a wave runs on as soon as
    // its part of the state has landed.
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    // ---- 3. X = S K~^T: K~ has 8 rows, so the tile's lanes m >= 8 repeat
    //      rows m - 8 and those columns of the result are dropped
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int bn = m & (kChunk - 1);
    if constexpr (kBf16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&Bh[bn][32 * c + 8 * g]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&Bl[bn][32 * c + 8 * g]);
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, fr[c][0]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int l = 0; l < 2; ++l) {
                const float4 bq = *reinterpret_cast<const float4 *>(&Bm[bn][32 * c + 8 * g + 4 * l]);
                const float bv4[4] = {bq.x, bq.y, bq.z, bq.w};
                const uint32_t w4[4] = {fr[c][l].x, fr[c][l].y, fr[c][l].z, fr[c][l].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w4[e]), bv4[e], acc, 0, 0, 0);
            }
    }
    if (m < kChunk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Xs[16 * wave + 4 * g + r][m] = acc[r];
    }
    wave_sync();

    // ---- 4. per value row r of the wave: the d recurrence
    if (lane < 16) {
        const int r = 16 * wave + lane;
        float d[kChunk];
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            d[t] = 0.f;
            if (t < na) {
                float u = Xs[r][t];
#pragma unroll
                for (int jj = 0; jj < t; ++jj) u = fmaf(Am[t][jj] * nk[t] * nk[jj], d[jj], u);
                d[t] = bsh[t] * (vs[t][r] - u);
                Ds[t][r] = d[t];
            }
        }
    }
    wave_sync();

    // ---- 5. S_na = S e^{G_na} + sum_t d_t KD_t^T, per (column block, half)
    {
        float sv[4][8];  // the lane's state elements in fp32
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (kBf16) {
                Stor<bf16_t>::unpack(fr[c][0], sv[c]);
            } else {
                Stor<float>::unpack(fr[c][0], sv[c]);
                Stor<float>::unpack(fr[c][1], sv[c] + 4);
            }
        }
        const int row = 16 * wave + m;
        const float d_lo = Ds[g][row], d_hi = Ds[4 + g][row];  // B operand: d_{g}, d_{4+g} of row m
        float out[4][8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 e0 = *reinterpret_cast<const float4 *>(&Ee[32 * c + 8 * g]);
            const float4 e1 = *reinterpret_cast<const float4 *>(&Ee[32 * c + 8 * g + 4]);
            const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 u;
#pragma unroll
                for (int r = 0; r < 4; ++r) u[r] = sv[c][4 * hf + r] * ev[4 * hf + r];
                // A operand: lane (m, g) supplies KD_t[col(m)] for t = g (then 4 + g)
                const int colm = 32 * c + 8 * (m >> 2) + 4 * hf + (m & 3);
                u = __builtin_amdgcn_mfma_f32_16x16x4f32(KD[g][colm], d_lo, u, 0, 0, 0);
                u = __builtin_amdgcn_mfma_f32_16x16x4f32(KD[4 + g][colm], d_hi, u, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) out[c][4 * hf + r] = u[r];
            }
        }
        char *Sw = const_cast<char *>(Srow);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (kBf16) {
                st_stream(Sw + (int64_t)(32 * c + 8 * g) * 2, Stor<bf16_t>::pack(out[c]));
            } else {
                st_stream(Sw + (int64_t)(32 * c + 8 * g) * 4, Stor<float>::pack(out[c]));
                st_stream(Sw + (int64_t)(32 * c + 8 * g) * 4 + 16, Stor<float>::pack(out[c] + 4));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fast rebuild (ring fold)
// ---------------------------------------------------------------------------
// S_m = S_0 Diag(exp(G_m)) + sum_j d_j (k_j . exp(G_m - G_j))^T with G_j the
// cumulative log decay of the first j folded steps: the unrolled sum of the
// ReplaySSM d/k/g passage, 16 steps per LDS pass (passes compose).
constexpr int kFold = 16;
// One pass of the fold over nc <= kFold ring steps from step t0.  Staging:
// the records as 16-byte loads, d and k in units of V16<IOT>::N values, the
// gates in units of four channels (GDN: the step's gate four times).
// Indices are clamped, so every load is issued with no branch; rows past
// the pass's last step repeat it and are never read.
template <typename IOT, bool KDA, int NT> struct FoldStage {
    static constexpr int VI = V16<IOT>::N, ND = kFold * HD / VI, NG = kFold * HD / 4;
    static constexpr int UD = (ND + NT - 1) / NT, UG = (NG + NT - 1) / NT;
    uint4 d[UD], k[UD], g[UG];

    __device__ __forceinline__ void load(const FoldArgs &a, int slot, int h, int rb, int t0, int nc,
                                         int tid)
    {
        const RingArgs &R = a.ring;
#pragma unroll
        for (int q = 0; q < UD; ++q) {
            const int e = min(tid + q * NT, ND - 1) * VI;
            const int pos = (rb + t0 + min(e / HD, nc - 1)) & (R.L - 1);
            const int64_t vr = ring_at(slot, a.Hv, R.L, h, pos, HD) + e % HD;
            d[q] = *reinterpret_cast<const uint4 *>(static_cast<const IOT *>(R.d) + vr);
            k[q] = *reinterpret_cast<const uint4 *>(static_cast<const IOT *>(R.k) + vr);
        }
#pragma unroll
        for (int q = 0; q < UG; ++q) {
            const int e = min(tid + q * NT, NG - 1) * 4;
            const int pos = (rb + t0 + min(e / HD, nc - 1)) & (R.L - 1);
            if constexpr (KDA) {
                g[q] = *reinterpret_cast<const uint4 *>(R.g + ring_at(slot, a.Hv, R.L, h, pos, HD) + e % HD);
            } else {
                const uint32_t g1 = __float_as_uint(R.g[ring_at(slot, a.Hv, R.L, h, pos, 1)]);
                g[q] = make_uint4(g1, g1, g1, g1);
            }
        }
    }

    // The staged records to LDS, then per channel the cumulative decay and
    // the decayed keys; starts and ends with a barrier.
    __device__ __forceinline__ void tables(float (*dsh)[HD], float (*esh)[HD], float (*gsh)[HD],
                                           float *eend, int nc, int tid) const
    {
        __syncthreads();  // the previous pass's tables are no longer read
#pragma unroll
        for (int q = 0; q < UD; ++q) {
            const int u = tid + q * NT;
            if (u < ND) {
                const int t = u * VI / HD, c = u * VI % HD;
                float v[VI];
                unpack16<IOT>(d[q], v);
#pragma unroll
                for (int e = 0; e < VI; e += 4)
                    *reinterpret_cast<float4 *>(&dsh[t][c + e]) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
                unpack16<IOT>(k[q], v);
#pragma unroll
                for (int e = 0; e < VI; e += 4)
                    *reinterpret_cast<float4 *>(&esh[t][c + e]) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
            }
        }
#pragma unroll
        for (int q = 0; q < UG; ++q) {
            const int u = tid + q * NT;
            if (u < NG) *reinterpret_cast<uint4 *>(&gsh[4 * u / HD][4 * u % HD]) = g[q];
        }
        __syncthreads();
        if (tid < HD) {  // per channel: running sums (floored gates), decayed keys
            float G = 0.f;
            for (int t = 0; t < nc; ++t) {
                G += fmaxf(gsh[t][tid], kGFloor);
                gsh[t][tid] = G;
            }
            eend[tid] = fast_exp(G);
            for (int t = 0; t < nc; ++t) esh[t][tid] *= fast_exp(G - gsh[t][tid]);
        }
        __syncthreads();
    }
};

template <typename ST, typename IOT, bool KDA, bool PROJ>
__global__ void __launch_bounds__((DecodeCfg<HD, ST>::NT)) fold_kernel(FoldArgs a)
{
    using Cfg = DecodeCfg<HD, ST>;
    constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPW = Cfg::RPW, NJ = Cfg::NJ, NT = Cfg::NT;
    __shared__ __align__(16) float dsh[kFold][HD];  // d_j
    __shared__ __align__(16) float esh[kFold][HD];  // k_j, then k_j exp(G_end - G_j)
    __shared__ __align__(16) float gsh[kFold][HD];  // g_j, then G_j
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
    const int col0 = (lane % LPR) * EPL;
    const int rb = a.ring_base[b];
    float s[NJ][EPL];
    // s = s Diag(exp(G_end)) + sum_t d_t (k_t exp(G_end - G_t))^T over a pass
    auto apply = [&](int nc) {
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
    };
    // First pass: its records go out first and the state rows right behind
    // them (loads complete in issue order, so waiting for the records does
    // not wait for the rows); the rows are unpacked only once the tables are
    // built, so they land under the staging.  With m = 0 the records loaded
    // are unused and the checkpoint is copied.
    const int nc0 = min(kFold, m);
    {
        uint4 raw[NJ];
        FoldStage<IOT, KDA, NT> fs;
        fs.load(a, slot, h, rb, 0, max(nc0, 1), tid);
        __builtin_amdgcn_sched_barrier(0);
        load_rows<HD, ST>(raw, S0, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (m > 0) fs.tables(dsh, esh, gsh, eend, nc0, tid);
#pragma unroll
        for (int j = 0; j < NJ; ++j) Stor<ST>::unpack(raw[j], s[j]);
    }
    if (m > 0) apply(nc0);
    for (int t0 = kFold; t0 < m; t0 += kFold) {
        const int nc = min(kFold, m - t0);
        FoldStage<IOT, KDA, NT> fs;
        fs.load(a, slot, h, rb, t0, nc, tid);
        fs.tables(dsh, esh, gsh, eend, nc, tid);
        apply(nc);
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
    const dim3 grid((unsigned)(a.B * a.Hv));
    if (a.D <= kChunk) {  // one chunk: the matrix-core form
        if (a.w)
            hipLaunchKernelGGL((verify_chunk_kernel<ST, IOT, CT, KDA, true>), grid, dim3(kChunkNT), 0, stream, a);
        else
            hipLaunchKernelGGL((verify_chunk_kernel<ST, IOT, CT, KDA, false>), grid, dim3(kChunkNT), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 block(DecodeCfg<HD, ST>::NT);
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
                       dim3(kCommitNT), 0, stream, a);
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
