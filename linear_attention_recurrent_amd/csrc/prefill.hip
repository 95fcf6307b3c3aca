// prefill.hip -- chunked prefill of the gated delta rule (KDA per-channel
// decay, GDN scalar decay) over packed variable-length sequences.
//
// The pages describe extend as a chunk-parallel algorithm with block 64: the
// state is read from the pool, blocks combine an inter-block recurrence with
// intra-block parallel work, and the final state is written back in place
// ("SGLang之KV Cache内存池机制", section 8.5, forward_extend).  The algebra
// below follows from the unrolled form of the recurrence printed in the
// ReplaySSM fast-rebuild passage of xxmr.cn/news/181459:
//     S_t = S_0 Diag(Gamma_t) + sum_{j<=t} d_j (k_j . Gamma_t / Gamma_j)^T.
//
// Per block of L <= 64 tokens of one sequence and value head, with q, k
// L2-normalised, G_t the cumulative log decay (per key channel) and
// Gamma_t = exp(G_t - G_start):
//   A_tj = sum_c k_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j < t)
//   P_tj = sum_c q_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j <= t)
//   T    = (I + Diag(beta) A)^-1                        unit lower triangular
//   U    = T Diag(beta) V,   W = T Diag(beta) (K . Gamma)
//   D    = U - W S_0^T                                  rows d_t of the recurrence
//   O    = scale ((Q . Gamma) S_0^T + P D)
//   S_L  = S_0 Diag(Gamma_L) + D^T (K . Gamma_L / Gamma)
// U, W, P and the scaled Q, K do not depend on S_0: kernel 1 computes them for
// every block in parallel; kernel 2 runs the block chain per (sequence, head,
// 16-row slice of the state), rows of S being independent given the block.
//
// Blocks are the intersections of 64-token tiles of the packed token axis
// with the sequences ("pieces").  Kernel 1 works per (tile, head) with a
// same-sequence mask on A and P, so one launch covers every sequence; the
// cumulative decay G runs continuously over the tile and only differences of
// G between tokens of one piece enter the results.  Kernel 2 walks a
// sequence's tiles and treats each piece as the full 64-token tile with the
// other rows masked to zero, so every access stays tile-aligned.
//
// Overflow-safe factorisation of A and P.  For row sub-block I (tokens
// 16I..16I+15) the reference R_I = G_{16I-1} (0 for I = 0) splits
//   exp(G_t - G_j) = exp(G_t - R_I) exp(R_I - G_j)
// with both factors <= 1 whenever j < 16I <= t, so the off-diagonal 16x16
// tiles are plain matrix products.  On the diagonal tile the j-side factor is
// >= 1 and bounded by exp of the decay accumulated over 16 tokens; exponents
// are clamped at 80 (e^80 ~ 5.5e34), which is exact while that accumulated
// decay stays below 80 (an average |g| < 5 per token).
//
// Matrix cores.  Every contraction is an "NT" product C[i][j] =
// sum_k A[i][k] B[j][k] of 16x16 output tiles with both operands row-major
// over k.  Two precisions (the `mode` argument):
//   fp32    v_mfma_f32_16x16x4f32; lane (i, q) of a tile owns the contiguous
//           k range [q K/4, (q+1) K/4) and step m uses k = q K/4 + m;
//   bf16x3  v_mfma_f32_16x16x32_bf16 on a two-term bf16 split of each
//           operand, a = a_hi + a_lo, accumulating a_lo b_hi + a_hi b_lo +
//           a_hi b_hi in fp32 (the dropped a_lo b_lo is ~2^-16 relative);
//           step s uses k = 32 s + 8 q + e, e < 8 (layouts checked on gfx950).
// (bf16-rounded operands alone were measured at up to 3e-2 per-unit error on
// the outputs, from cancellation in the contractions, and are not offered.)
// The result tile D[4 (l/16) + r][l % 16] sits in register r of lane l.
// The small 16x16 block products of the triangular inverse always use fp32.
#include "la_device.h"
#include "la_internal.h"

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int CB = 64;         // tokens per tile
constexpr int DK = 128;        // head dim (d_k = d_v)
constexpr int LDK = DK + 8;    // LDS row stride (floats) of [64 x 128] arrays (16-byte rows)
constexpr int LDJ = CB + 4;    // LDS row stride of [* x 64] arrays
constexpr float kExpClamp = 80.f;
enum { PM_F32 = 0, PM_BF16X3 = 1 };

// exp(x) as 2^(x log2 e) with the product carried in two pieces before the
// hardware exp2: about 2 ulp for the |x| <= 88 used here.
__device__ __forceinline__ float exp_acc(float x)
{
    const float kHi = 1.44269502162933349609375f, kLo = 1.925963033500011e-8f;
    const float t = x * kHi;
    float e = fmaf(x, kHi, -t);
    e = fmaf(x, kLo, e);
    return __builtin_amdgcn_exp2f(t) * fmaf(e, 0.69314718f, 1.0f);
}

// ---- NT fragments ---------------------------------------------------------
// A lane's fragment of one operand row for a K-long contraction holds K/4
// floats; element idx corresponds to k = frag_k(q, idx).
template <int MODE, int K> __device__ __forceinline__ int frag_k(int q, int idx)
{
    if constexpr (MODE == PM_F32) return q * (K / 4) + idx;
    else return 32 * (idx >> 3) + 8 * q + (idx & 7);
}
// Offset of the lane's 4-float group g (g < K/16) inside the row.
template <int MODE, int K> __device__ __forceinline__ int frag_off4(int q, int g)
{
    if constexpr (MODE == PM_F32) return q * (K / 4) + 4 * g;
    else return 32 * (g >> 1) + 8 * q + 4 * (g & 1);
}
template <int MODE, int K>
__device__ __forceinline__ void load_frag(float *fr, const float *row, int q)
{
#pragma unroll
    for (int g = 0; g < K / 16; ++g) {
        const float4 v = *reinterpret_cast<const float4 *>(row + frag_off4<MODE, K>(q, g));
        fr[4 * g] = v.x; fr[4 * g + 1] = v.y; fr[4 * g + 2] = v.z; fr[4 * g + 3] = v.w;
    }
}

__device__ __forceinline__ bf16x8_t to_bf16x8(const float *f)
{
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e];
    return __builtin_convertvector(v, bf16x8_t);
}
__device__ __forceinline__ bf16x8_t lo_bf16x8(const float *f, bf16x8_t hi)
{
    const f32x8 back = __builtin_convertvector(hi, f32x8);
    f32x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f[e] - back[e];
    return __builtin_convertvector(v, bf16x8_t);
}

// Elements a lane supplies per instruction, and the k consumed per instruction.
template <int MODE> struct Step {
    static constexpr int W = MODE == PM_F32 ? 1 : 8;
    static constexpr int K = MODE == PM_F32 ? 4 : 32;
};

// One matrix-core step: acc += A_step B_step^T from this lane's W elements.
template <int MODE>
__device__ __forceinline__ void mma_step(f32x4 &acc, const float *a, const float *b)
{
    if constexpr (MODE == PM_F32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    } else {
        const bf16x8_t ah = to_bf16x8(a), bh = to_bf16x8(b);
        const bf16x8_t al = lo_bf16x8(a, ah), bl = lo_bf16x8(b, bh);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    }
}

// acc += A B^T over K.  fa(idx, k) / fb(idx, k) return this lane's operand
// element for fragment index idx, which covers contraction index
// k = frag_k(q, idx): a register fragment ignores k, an LDS row ignores idx.
template <int MODE, int K, class FA, class FB>
__device__ __forceinline__ void mma_gen(f32x4 &acc, int q, FA fa, FB fb)
{
    constexpr int W = Step<MODE>::W;
#pragma unroll
    for (int m = 0; m < K / Step<MODE>::K; ++m) {
        float av[W], bv[W];
#pragma unroll
        for (int e = 0; e < W; ++e) {
            const int idx = m * W + e, k = frag_k<MODE, K>(q, idx);
            av[e] = fa(idx, k);
            bv[e] = fb(idx, k);
        }
        mma_step<MODE>(acc, av, bv);
    }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- workspace -------------------------------------------------------------
// fp32 arrays indexed by (token, value head): U, W, Q Gamma [.., 128],
// P [.., 64] (tile-local columns), the piece's total log decay [.., 128] (at
// piece-end tokens); and K Gamma_L / Gamma transposed per (tile, head):
// [128 channels][64 tokens].
struct Ws {
    float *U, *W, *Qt, *P, *Ge, *KhT;
};
__host__ __device__ inline Ws ws_layout(void *base, int T, int Hv)
{
    const size_t n = (size_t)T * Hv;
    float *p = static_cast<float *>(base);
    Ws w;
    w.U = p;
    w.W = w.U + n * DK;
    w.Qt = w.W + n * DK;
    w.Ge = w.Qt + n * DK;
    w.P = w.Ge + n * DK;
    w.KhT = w.P + n * CB;
    return w;
}

size_t prefill_ws_bytes(int N, int T, int Hqk, int Hv, int D, int mode)
{
    (void)N; (void)Hqk; (void)mode;
    if (D != DK || T <= 0) return 0;
    const size_t tiles = (size_t)(T + CB - 1) / CB;
    const size_t floats = (size_t)T * Hv * (4 * DK + CB) + tiles * Hv * DK * CB;
    return (floats * sizeof(float) + 255) & ~size_t(255);
}

__device__ __forceinline__ int find_seq_p(const int32_t *cu, int N, int t)
{
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Loads 16 consecutive elements of type T as floats.
template <typename T> __device__ __forceinline__ void load16(float *f, const void *p);
template <> __device__ __forceinline__ void load16<float>(float *f, const void *p)
{
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 v = static_cast<const float4 *>(p)[g];
        f[4 * g] = v.x; f[4 * g + 1] = v.y; f[4 * g + 2] = v.z; f[4 * g + 3] = v.w;
    }
}
template <> __device__ __forceinline__ void load16<bf16_t>(float *f, const void *p)
{
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const uint4 v = static_cast<const uint4 *>(p)[g];
        f[8 * g] = bf16_lo(v.x); f[8 * g + 1] = bf16_hi(v.x);
        f[8 * g + 2] = bf16_lo(v.y); f[8 * g + 3] = bf16_hi(v.y);
        f[8 * g + 4] = bf16_lo(v.z); f[8 * g + 5] = bf16_hi(v.z);
        f[8 * g + 6] = bf16_lo(v.w); f[8 * g + 7] = bf16_hi(v.w);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-block quantities, one workgroup (8 waves) per (tile, head).
// ---------------------------------------------------------------------------
constexpr int kIntraThreads = 512;
constexpr size_t kIntraLdsFloats = 3 * CB * LDK + 2 * CB * LDJ + CB + 4 * DK + 8 * 16 * 17;
constexpr size_t kIntraLds = kIntraLdsFloats * sizeof(float) + 2 * CB * sizeof(int);

template <typename IOT, bool KDA, int MODE>
__global__ void __launch_bounds__(kIntraThreads) prefill_intra_kernel(PrefillArgs a)
{
    extern __shared__ float sm[];
    float *Qn = sm;                  // q_hat [64][LDK]; later (beta K Gamma)^T [128][LDJ]
    float *Kn = Qn + CB * LDK;       // k_hat [64][LDK]; later (beta V)^T [128][LDJ]
    float *Gc = Kn + CB * LDK;       // cumulative log decay over the tile
    float *Nm = Gc + CB * LDK;       // N = Diag(beta) A (strictly lower, masked); earlier K^ T
    float *Tm = Nm + CB * LDJ;       // T = (I + N)^-1
    float *bet = Tm + CB * LDJ;      // beta
    float *qsum = bet + CB;          // [4][128] partial sums of the tile scan
    float *scr = qsum + 4 * DK;      // per-wave 16x17 scratch
    int *pst = reinterpret_cast<int *>(scr + 8 * 16 * 17);  // piece start (tile-local)
    int *pen = pst + CB;                                      // piece end (inclusive)
    float *XtK = Qn, *XtV = Kn;      // transposed right-hand sides of phase 6
    float *KhTl = Nm;                // [128][LDJ] staging of K Gamma_L / Gamma, transposed

    const int tile = blockIdx.x, h = blockIdx.y, kh = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int t0 = tile * CB;
    const int nt = min(CB, a.T - t0);
    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    auto row = [&](int t) { return ((int64_t)(t0 + t) * a.Hv + h); };

    // ---- 1. loads: thread (token t, 16-channel chunk cq), all issued up front
    const int t = tid >> 3, cq = tid & 7, c0 = 16 * cq;
    const bool valid = t < nt;
    const int64_t tok = t0 + min(t, nt - 1);
    float qv[16], kv[16], gv[16];
    load16<IOT>(qv, static_cast<const IOT *>(a.q) + tok * a.q_stride + kh * DK + c0);
    load16<IOT>(kv, static_cast<const IOT *>(a.k) + tok * a.k_stride + kh * DK + c0);
    if constexpr (KDA) {
        load16<float>(gv, a.g + (tok * a.Hv + h) * DK + c0);
    } else {
        const float g1 = a.g[tok * a.Hv + h];
#pragma unroll
        for (int e = 0; e < 16; ++e) gv[e] = g1;
    }
    const float bt = a.beta[tok * a.Hv + h];
    int ps = t, pe = t;
    if (valid) {
        const int n = find_seq_p(a.cu, a.N, t0 + t);
        ps = max(a.cu[n], t0) - t0;
        pe = min(a.cu[n + 1], t0 + CB) - 1 - t0;
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (!valid) { qv[e] = 0.f; kv[e] = 0.f; gv[e] = 0.f; }
        sq = fmaf(qv[e], qv[e], sq);
        sk = fmaf(kv[e], kv[e], sk);
    }
    sq = group_sum<8>(sq);
    sk = group_sum<8>(sk);
    const float iq = 1.f / sqrtf(sq + a.eps), ik = 1.f / sqrtf(sk + a.eps);
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
        *reinterpret_cast<float4 *>(Qn + t * LDK + c0 + e) =
            make_float4(qv[e] * iq, qv[e + 1] * iq, qv[e + 2] * iq, qv[e + 3] * iq);
        *reinterpret_cast<float4 *>(Kn + t * LDK + c0 + e) =
            make_float4(kv[e] * ik, kv[e + 1] * ik, kv[e + 2] * ik, kv[e + 3] * ik);
        *reinterpret_cast<float4 *>(Gc + t * LDK + c0 + e) =
            make_float4(gv[e], gv[e + 1], gv[e + 2], gv[e + 3]);
    }
    if (cq == 0) {
        bet[t] = valid ? bt : 0.f;
        pst[t] = ps;
        pen[t] = pe;
    }
    __syncthreads();

    // ---- 2. cumulative decay over the tile: 4 quarters of 16 tokens per channel
    {
        const int c = tid & (DK - 1), qq = tid >> 7;
        float run[16];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc += Gc[(16 * qq + i) * LDK + c];
            run[i] = acc;
        }
        qsum[qq * DK + c] = acc;
        __syncthreads();
        float off = 0.f;
        for (int p = 0; p < qq; ++p) off += qsum[p * DK + c];
#pragma unroll
        for (int i = 0; i < 16; ++i) Gc[(16 * qq + i) * LDK + c] = run[i] + off;
    }
    __syncthreads();

    // ---- 3. Q Gamma (global), the piece's total decay (global, at piece ends),
    //         K Gamma_L / Gamma transposed through LDS
    {
        float qt[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int c = c0 + e;
            const float G = Gc[t * LDK + c];
            const float Gs = ps > 0 ? Gc[(ps - 1) * LDK + c] : 0.f;
            const float Ge = Gc[pe * LDK + c];
            qt[e] = Qn[t * LDK + c] * exp_acc(G - Gs);
            KhTl[c * LDJ + t] = Kn[t * LDK + c] * exp_acc(Ge - G);
            if (valid && t == pe) ws.Ge[row(t) * DK + c] = Ge - Gs;
        }
        if (valid) {
#pragma unroll
            for (int e = 0; e < 16; e += 4)
                *reinterpret_cast<float4 *>(ws.Qt + row(t) * DK + c0 + e) =
                    make_float4(qt[e], qt[e + 1], qt[e + 2], qt[e + 3]);
        }
    }
    __syncthreads();
    {   // KhT: [128][64] per (tile, head); thread (channel c, 16 tokens)
        const int c = tid >> 2, tq = 16 * (tid & 3);
        float *dst = ws.KhT + (((int64_t)tile * a.Hv + h) * DK + c) * CB + tq;
#pragma unroll
        for (int e = 0; e < 16; e += 4)
            *reinterpret_cast<float4 *>(dst + e) = *reinterpret_cast<const float4 *>(KhTl + c * LDJ + tq + e);
    }
    __syncthreads();
    for (int i = tid; i < 2 * CB * LDJ; i += kIntraThreads) Nm[i] = 0.f;  // Nm and Tm
    __syncthreads();

    // ---- 4. A and P, one 16x16 tile pair (I, J <= I) per wave job
    for (int job = wave; job < 10; job += 8) {
        // jobs in order of cost: (3,0..3), (2,0..2), (1,0..1), (0,0)
        const int I = job < 4 ? 3 : job < 7 ? 2 : job < 9 ? 1 : 0;
        const int J = job < 4 ? job : job < 7 ? job - 4 : job < 9 ? job - 7 : 0;
        const int ti = 16 * I + li, tj = 16 * J + li;
        constexpr int W = Step<MODE>::W;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
#pragma unroll
        for (int m = 0; m < DK / Step<MODE>::K; ++m) {
            float fk[W], fq[W], fj[W];
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const int c = frag_k<MODE, DK>(lq, m * W + e);
                const float R = I ? Gc[(16 * I - 1) * LDK + c] : 0.f;
                const float et = exp_acc(fminf(Gc[ti * LDK + c] - R, kExpClamp));
                fk[e] = Kn[ti * LDK + c] * et;
                fq[e] = Qn[ti * LDK + c] * et;
                fj[e] = Kn[tj * LDK + c] * exp_acc(fminf(R - Gc[tj * LDK + c], kExpClamp));
            }
            mma_step<MODE>(accA, fk, fj);
            mma_step<MODE>(accP, fq, fj);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tt = 16 * I + 4 * lq + r, j = 16 * J + li;
            const bool same = j >= pst[tt] && tt < nt;
            Nm[tt * LDJ + j] = (same && j < tt) ? bet[tt] * accA[r] : 0.f;
            if (tt < nt) ws.P[row(tt) * CB + j] = (same && j <= tt) ? accP[r] : 0.f;
        }
    }
    for (int idx = tid; idx < nt * CB; idx += kIntraThreads) {  // upper tiles of P are zero
        const int tt = idx / CB, j = idx % CB;
        if ((j >> 4) > (tt >> 4)) ws.P[row(tt) * CB + j] = 0.f;
    }
    __syncthreads();

    // ---- 5. T = (I + N)^-1: diagonal 16x16 blocks by forward substitution
    //         (waves 0..3, lane c < 16 holds column c), then the off-diagonal
    //         blocks level by level: T_IJ = -T_II sum_{K=J}^{I-1} N_IK T_KJ.
    if (wave < 4 && lane < 16) {
        const int I = wave, c = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) s = fmaf(Nm[(16 * I + r) * LDJ + 16 * I + j], x[j], s);
            x[r] = r == c ? 1.f : (r < c ? 0.f : -s);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[(16 * I + r) * LDJ + 16 * I + c] = x[r];
    }
    __syncthreads();
    float *ws16 = scr + wave * 16 * 17;
    for (int lev = 1; lev <= 3; ++lev) {
        const int I = wave, J = wave - lev;
        if (wave < 4 && J >= 0) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K)
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma4(Nm[(16 * I + li) * LDJ + 16 * K + k0 + lq],
                                Tm[(16 * K + k0 + lq) * LDJ + 16 * J + li], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) ws16[(4 * lq + r) * 17 + li] = acc[r];
            __builtin_amdgcn_wave_barrier();
            f32x4 t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += 4)
                t2 = mfma4(Tm[(16 * I + li) * LDJ + 16 * I + k0 + lq], ws16[(k0 + lq) * 17 + li], t2);
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(16 * I + 4 * lq + r) * LDJ + 16 * J + li] = -t2[r];
        }
        __syncthreads();
    }

    // ---- 6. right-hand sides, transposed: (beta K Gamma)^T and (beta V)^T
    {
        const int c = tid & (DK - 1), tq = 16 * (tid >> 7);
        float xk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tt = tq + i;
            const float Gs = pst[tt] > 0 ? Gc[(pst[tt] - 1) * LDK + c] : 0.f;
            xk[i] = bet[tt] * Kn[tt * LDK + c] * exp_acc(Gc[tt * LDK + c] - Gs);
        }
        __syncthreads();  // Qn is about to be overwritten
#pragma unroll
        for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<float4 *>(XtK + c * LDJ + tq + i) =
                make_float4(xk[i], xk[i + 1], xk[i + 2], xk[i + 3]);
    }
    {
        float vv[16];
        load16<IOT>(vv, static_cast<const IOT *>(a.v) + tok * a.v_stride + h * DK + c0);
        __syncthreads();  // Kn is free
#pragma unroll
        for (int e = 0; e < 16; ++e) XtV[(c0 + e) * LDJ + t] = valid ? bet[t] * vv[e] : 0.f;
    }
    __syncthreads();

    // ---- 7. U = T (beta V) and W = T (beta K Gamma): wave w owns output
    //         columns 16w .. 16w + 15 of both, for the four token blocks
    {
        const int C = wave;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const float *Xt = which ? XtK : XtV;
            float *dst = which ? ws.W : ws.U;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const float *Trow = Tm + (16 * I + li) * LDJ, *Xrow = Xt + (16 * C + li) * LDJ;
                auto fa = [&](int, int j) { return Trow[j]; };
                auto fb = [&](int, int j) { return Xrow[j]; };
                if (I < 2) mma_gen<MODE, 32>(acc, lq, fa, fb);  // T rows < 32: columns < 32
                else mma_gen<MODE, 64>(acc, lq, fa, fb);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = 16 * I + 4 * lq + r;
                    if (tt < nt) dst[row(tt) * DK + 16 * C + li] = acc[r];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: the block chain, one workgroup per (sequence, head, 16 state rows).
// Waves 0..3 ("row waves") own token rows 16I.. of D and O; waves 4..7
// ("column waves") own state columns 32(w-4) .. 32(w-4) + 31 of the update.
// The next tile's W, U (row waves) and K^T, Gamma (column waves) are loaded
// into registers while the current tile computes.
// ---------------------------------------------------------------------------
constexpr int kChainThreads = 512;
constexpr size_t kChainLds = (16 * LDK + 16 * LDJ) * sizeof(float);

// Per-lane prefetch buffer, shared by the two wave roles:
//   row waves:    [0, 32) W row fragment (K = 128 channels), [32, 36) U values;
//   column waves: [0, 32) K^T row fragments of two column tiles (K = 64
//                 tokens, 16 each), [32, 34) Gamma_L of the lane's columns.
constexpr int kOps = 36;

template <typename IOT, typename ST, int MODE>
__global__ void __launch_bounds__(kChainThreads) prefill_chain_kernel(PrefillArgs a)
{
    extern __shared__ float sm[];
    float *St = sm;               // state slice [16 rows][LDK]
    float *Dt = St + 16 * LDK;    // D^T of the tile [16 rows][LDJ] (tile-local tokens)

    const int n = blockIdx.x, h = blockIdx.y, rs = blockIdx.z;  // rows 16 rs .. 16 rs + 15
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const bool rowwave = wave < 4;
    const int I = wave & 3;       // token block (row waves) / column pair (column waves)
    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    const int start = a.cu[n], end = a.cu[n + 1];
    const int si = a.slot_in[n], so = a.slot_out[n];

    if (si >= a.num_rows || so < 0 || so >= a.num_rows) {  // skipped sequence
        for (int idx = tid; idx < (end - start) * 16; idx += kChainThreads) {
            const int t = start + idx / 16, c = 16 * rs + idx % 16;
            st<IOT>(a.out, ((int64_t)t * a.Hv + h) * DK + c, 0.f);
        }
        return;
    }
    for (int idx = tid; idx < 16 * DK; idx += kChainThreads) {  // initial state slice
        const int i = idx / DK, c = idx % DK;
        float v = 0.f;
        if (si >= 0)
            v = ld<ST>(a.ssm_pool,
                       (int64_t)si * a.ssm_stride + ((int64_t)h * DK + 16 * rs + i) * DK + c);
        St[i * LDK + c] = v;
    }

    const int tb0 = start / CB, tb1 = end > start ? (end - 1) / CB : tb0 - 1;
    // Operand prefetch for tile tb (clamped: loads stay inside the arrays).
    auto load_ops = [&](int tb, float *ops) {
        const int base = tb * CB;
        if (rowwave) {
            const int tt = min(base + 16 * I + li, a.T - 1);
            load_frag<MODE, DK>(ops, ws.W + ((int64_t)tt * a.Hv + h) * DK, lq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = min(base + 16 * I + 4 * lq + r, a.T - 1);
                ops[32 + r] = ws.U[((int64_t)tr * a.Hv + h) * DK + 16 * rs + li];
            }
        } else {
            const int pend = min(end, base + CB) - 1;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = 32 * I + 16 * q + li;
                load_frag<MODE, CB>(ops + 16 * q, ws.KhT + (((int64_t)tb * a.Hv + h) * DK + c) * CB, lq);
                ops[32 + q] = ws.Ge[((int64_t)max(pend, 0) * a.Hv + h) * DK + c];
            }
        }
    };

    float cur[kOps], nxt[kOps];
    if (tb1 >= tb0) load_ops(tb0, cur);
    for (int tb = tb0; tb <= tb1; ++tb) {
        const int base = tb * CB;
        const int p0 = max(start, base) - base, p1 = min(end, base + CB) - base;
        load_ops(min(tb + 1, tb1), nxt);  // next tile (the last one reloads itself)
        __syncthreads();                   // state of the previous tile in place

        float fq[DK / 4], fp[CB / 4];
        const float *Srow = St + li * LDK, *Drow = Dt + li * LDJ;
        auto lds_s = [&](int, int c) { return Srow[c]; };
        auto lds_d = [&](int, int j) { return Drow[j]; };
        if (rowwave) {
            // D = U - W S^T, rows outside the piece masked
            const int ti = 16 * I + li;
            const bool in_i = ti >= p0 && ti < p1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_gen<MODE, DK>(acc, lq, [&](int idx, int) { return in_i ? cur[idx] : 0.f; }, lds_s);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * I + 4 * lq + r;
                const bool in_r = tr >= p0 && tr < p1;
                Dt[li * LDJ + tr] = in_r ? cur[32 + r] - acc[r] : 0.f;
            }
            // Q Gamma and P rows for the output (off the chain's critical path)
            const int tt = min(base + ti, a.T - 1);
            load_frag<MODE, DK>(fq, ws.Qt + ((int64_t)tt * a.Hv + h) * DK, lq);
            load_frag<MODE, CB>(fp, ws.P + ((int64_t)tt * a.Hv + h) * CB, lq);
        }
        __syncthreads();  // D^T complete

        f32x4 snew[2];
        if (rowwave) {
            // O = scale (Q Gamma S^T + P D)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma_gen<MODE, DK>(acc, lq, [&](int idx, int) { return fq[idx]; }, lds_s);
            mma_gen<MODE, CB>(acc, lq, [&](int idx, int) { return fp[idx]; }, lds_d);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * I + 4 * lq + r;
                if (tr >= p0 && tr < p1)
                    st<IOT>(a.out, ((int64_t)(base + tr) * a.Hv + h) * DK + 16 * rs + li,
                            a.scale * acc[r]);
            }
        } else {
            // new state columns: S Gamma_L + D^T K^  (K^ columns outside the piece masked)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                mma_gen<MODE, CB>(acc, lq, lds_d, [&](int idx, int j) {
                    return (j >= p0 && j < p1) ? cur[16 * q + idx] : 0.f;
                });
                const int c = 32 * I + 16 * q + li;
                const float gm = exp_acc(cur[32 + q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(St[(4 * lq + r) * LDK + c], gm, acc[r]);
                snew[q] = acc;
            }
        }
        __syncthreads();  // every wave done reading the old state
        if (!rowwave) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) St[(4 * lq + r) * LDK + 32 * I + 16 * q + li] = snew[q][r];
        }
#pragma unroll
        for (int i = 0; i < kOps; ++i) cur[i] = nxt[i];
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * DK; idx += kChainThreads) {
        const int i = idx / DK, c = idx % DK;
        st<ST>(a.ssm_pool, (int64_t)so * a.ssm_stride + ((int64_t)h * DK + 16 * rs + i) * DK + c,
               St[i * LDK + c]);
    }
}

template <typename IOT, typename ST, int MODE>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    static const bool attr_done = [] {  // opt in to more than 64 KB of LDS per workgroup
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, true, MODE>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIntraLds);
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, false, MODE>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIntraLds);
        return true;
    }();
    (void)attr_done;
    if (a.T > 0) {
        const dim3 g1((unsigned)((a.T + CB - 1) / CB), (unsigned)a.Hv);
        if (a.kda)
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, true, MODE>), g1, dim3(kIntraThreads),
                               kIntraLds, stream, a);
        else
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, false, MODE>), g1, dim3(kIntraThreads),
                               kIntraLds, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 g2((unsigned)a.N, (unsigned)a.Hv, (unsigned)(DK / 16));
    hipLaunchKernelGGL((prefill_chain_kernel<IOT, ST, MODE>), g2, dim3(kChainThreads), kChainLds,
                       stream, a);
    return hipGetLastError();
}

template <int MODE> static hipError_t launch_prefill_m(const PrefillArgs &a, hipStream_t stream)
{
    const int code = (a.io_dtype ? 2 : 0) | (a.state_dtype ? 1 : 0);
    switch (code) {
    case 0: return launch_prefill_t<float, float, MODE>(a, stream);
    case 1: return launch_prefill_t<float, bf16_t, MODE>(a, stream);
    case 2: return launch_prefill_t<bf16_t, float, MODE>(a, stream);
    default: return launch_prefill_t<bf16_t, bf16_t, MODE>(a, stream);
    }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.mode) {
    case PM_F32: return launch_prefill_m<PM_F32>(a, stream);
    case PM_BF16X3: return launch_prefill_m<PM_BF16X3>(a, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace la
