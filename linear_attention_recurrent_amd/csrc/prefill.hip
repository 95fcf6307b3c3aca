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
// slice of 16 or 64 state rows), rows of S being independent given the block.
//
// Blocks are the intersections of 64-token tiles of the packed token axis
// with the sequences ("pieces").  Kernel 1 works per (tile, head) with a
// same-sequence mask on A and P, so one launch covers every sequence.  The
// cumulative decay G is a segmented sum over the tile: it starts again from
// zero at every piece start, so a piece's decay factors never see another
// request's gates and their magnitude is that of the piece's own decay.
// A gate at or below -128 (exp underflows to 0 in fp32; -inf is a reset)
// empties those state channels at that token.  When every key channel of a
// token is reset (always so for GDN), the token starts a new "sub-piece":
// no pair across it interacts, the sum restarts from zero there, the state
// entering the tile reaches no token from it on, and the piece's decay of
// that state is zero.  A reset of some channels only is floored at -128 in
// those channels' sums, which keeps every difference finite and gives the
// same zero factors across it.  Kernel 2 walks a sequence's
// tiles and treats each piece as the full 64-token tile with the other rows
// masked to zero, so every access stays tile-aligned.
//
// Factorisation of A and P (KDA).  Row t of 16-token sub-block I takes the
// reference R_t = G_{16I-1} when its piece began before the sub-block and 0
// (the piece's own start) otherwise, and
//   exp(G_t - G_j) = exp(G_t - R_t) exp(R_t - G_j),
// where G_t - R_t <= 0 is the decay accumulated inside the sub-block.  Off
// the diagonal (j < 16I <= t, one piece) both factors are <= 1, so those
// 16x16 tiles are plain matrix products whatever the decay.  On the diagonal
// the j-side factor is >= 1, bounded by exp of the sub-block's largest
// in-block decay ("span").  Sub-blocks whose span stays within kSpanMax use
// the factorised product; the others (strong decay, resets) form
// exp(G_t - G_j) <= 1 per element instead, which is exact for any g <= 0.
// GDN has one decay per token and always scales per element.
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
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int CB = 64;         // tokens per tile
constexpr int DK = 128;        // head dim (d_k = d_v)
// LDS row strides are 4 (mod 32) floats: rows stay 16-byte aligned and the
// 16-byte fragment reads of 8 consecutive lanes (8 rows) cover all 32 banks.
constexpr int LDK = DK + 4;    // [* x 128] arrays
constexpr int LDJ = CB + 4;    // [* x 64] arrays
constexpr int kRegion = 128 * LDJ > CB * LDK ? 128 * LDJ : CB * LDK;  // one [64 x 128] or [128 x 64] array
// Largest in-sub-block decay taken by the factorised diagonal product:
// exp(-64) keeps the t-side factor and the low bf16 part of its split far
// above the fp32 subnormals.  kExpClamp only keeps factors of masked
// (cross-piece) pairs finite.
constexpr float kSpanMax = 64.f;
constexpr float kExpClamp = 80.f;
constexpr float kGateFloor = -128.f;  // exp(-128) == 0 in fp32
// exp(x) where on, else 0: the exponential is taken unconditionally (a masked
// lane's argument is replaced by one whose exponential is 0 in fp32), so the
// masked products of steps 3 and 6 compile to straight-line code.
__device__ __forceinline__ float exp_if(bool on, float x) { return exp_acc(on ? x : -200.f); }
enum { PM_F32 = 0, PM_BF16X3 = 1 };

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
// Loads n consecutive runs of 64 float4 (fragment-major storage): this lane's
// float4 of each run, into fr[4 g .. 4 g + 3].
__device__ __forceinline__ void load_run(float *fr, const float *base, int n, int lane)
{
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        if (g >= n) break;
        const float4 v = *reinterpret_cast<const float4 *>(base + (g * 64 + lane) * 4);
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
// The lo part: each hi word is read back as a float from its packed dword (the
// low word by a shift, the high word by a mask) rather than converted again.
__device__ __forceinline__ bf16x8_t lo_bf16x8(const float *f, bf16x8_t hi)
{
    const u32x4_t w = __builtin_bit_cast(u32x4_t, hi);
    f32x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = f[2 * i] - __uint_as_float(w[i] << 16);
        v[2 * i + 1] = f[2 * i + 1] - __uint_as_float(w[i] & 0xFFFF0000u);
    }
    return __builtin_convertvector(v, bf16x8_t);
}

// bf16x3 operands pre-split in memory: 8 fp32 values as a bf16 "hi" word
// quad and a bf16 "lo" word quad (hi + lo equals the value to about 2^-16).
__device__ __forceinline__ void split8(const float *f, uint4 &hi, uint4 &lo)
{
    const bf16x8_t h = to_bf16x8(f), l = lo_bf16x8(f, h);
    hi = __builtin_bit_cast(uint4, h);
    lo = __builtin_bit_cast(uint4, l);
}
// bf16x3 rows in LDS (row stride LDJ words): bf16 hi words 0..31 and lo words
// 32..63 hold columns 0..63.  Writes columns k0 .. k0 + 15 of one row.
__device__ __forceinline__ void store_row_split16(float *row, int k0, const float *v)
{
    uint4 h0, l0, h1, l1;
    split8(v, h0, l0);
    split8(v + 8, h1, l1);
    *reinterpret_cast<uint4 *>(row + k0 / 2) = h0;
    *reinterpret_cast<uint4 *>(row + k0 / 2 + 4) = h1;
    *reinterpret_cast<uint4 *>(row + 32 + k0 / 2) = l0;
    *reinterpret_cast<uint4 *>(row + 32 + k0 / 2 + 4) = l1;
}
// Writes the split 8-value group of step m of a lane into a fragment-major
// block: the hi quad to run 2m, the lo quad to run 2m + 1 (bf16x3 layout).
__device__ __forceinline__ void store_split(float *blk, int m, int lane, const float *v)
{
    uint4 hi, lo;
    split8(v, hi, lo);
    *reinterpret_cast<uint4 *>(blk + (2 * m * 64 + lane) * 4) = hi;
    *reinterpret_cast<uint4 *>(blk + ((2 * m + 1) * 64 + lane) * 4) = lo;
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

// The transposed tile of the same step: acc += B_step A_step^T, with the three
// bf16x3 products taken in mma_step's order (lo(a) hi(b), hi(a) lo(b),
// hi(a) hi(b)).  Lane (i, q) then holds row i of A's tile against columns
// 4q .. 4q + 3 of B's.
template <int MODE>
__device__ __forceinline__ void mma_step_t(f32x4 &acc, const float *a, const float *b)
{
    if constexpr (MODE == PM_F32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b[0], a[0], acc, 0, 0, 0);
    } else {
        const bf16x8_t ah = to_bf16x8(a), bh = to_bf16x8(b);
        const bf16x8_t al = lo_bf16x8(a, ah), bl = lo_bf16x8(b, bh);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, al, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl, ah, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, ah, acc, 0, 0, 0);
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
// Everything the block chain reads per (tile, value head), bh = tile * H_v + h,
// stored in fragment-major order: each run of 64 float4 is exactly what one
// wave-wide 16-byte load of the chain kernel reads, lane after lane, so every
// such load covers 1 KiB of contiguous memory.  With lane = 16 lq + li:
//   U  [bh][I 4][rs 8][lane][4]  U[16I + 4lq + r][16rs + li] (matrix-core result order)
//   W  [bh][I 4][g 8][lane][4]   W[16I + li][frag_off4<DK>(lq, g) + e]
//   Qt [bh][I 4][g 8][lane][4]   (Q Gamma)[16I + li][frag_off4<DK>(lq, g) + e]
//   P  [bh][I 4][g 4][lane][4]   P[16I + li][frag_off4<CB>(lq, g) + e]
//   KhT[bh][cg 8][g 4][lane][4]  (K Gamma_L / Gamma)^T[16cg + li][frag_off4<CB>(lq, g) + e]
// and, indexed by token, Ge [T][H_v][128]: the piece's total log decay, at
// piece-end tokens.  The fragment order depends on the precision mode.
constexpr int kBlkDK = CB * DK;  // floats of one [64 x 128] array per (tile, head)
constexpr int kBlkCB = CB * CB;  // floats of P per (tile, head)
struct Ws {
    float *U, *W, *Qt, *P, *KhT, *Ge;
};
__host__ __device__ inline Ws ws_layout(void *base, int T, int Hv)
{
    const size_t nb = (size_t)((T + CB - 1) / CB) * Hv;
    float *p = static_cast<float *>(base);
    Ws w;
    w.U = p;
    w.W = w.U + nb * kBlkDK;
    w.Qt = w.W + nb * kBlkDK;
    w.P = w.Qt + nb * kBlkDK;
    w.KhT = w.P + nb * kBlkCB;
    w.Ge = w.KhT + nb * kBlkDK;
    return w;
}
// Float offset of (group g, lane) inside a fragment-major run.
__device__ __forceinline__ int fidx(int g, int lane) { return (g * 64 + lane) * 4; }

size_t prefill_ws_bytes(int N, int T, int Hqk, int Hv, int D, int mode)
{
    (void)N; (void)Hqk; (void)mode;
    if (D != DK || T <= 0) return 0;
    const size_t nb = (size_t)((T + CB - 1) / CB) * Hv;
    const size_t floats = nb * (4 * kBlkDK + kBlkCB) + (size_t)T * Hv * DK;
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

// Fused short conv (pre-conv projections x [T, C]): conv + SiLU of channel ch
// for the 16 tile tokens tq .. tq + 15 (tile starting at global token t0).
// A token's window is rows tok - 3 .. tok of x; positions before its
// sequence's start sst[tt] come from conv pool row ssl[tt] (< 0: zeros).  The
// 19 rows slide along the thread's tokens, so every x element is loaded once
// and the loads are coalesced over channels.  Tap order and sum order are
// those of the standalone conv kernels.  The caller's wave shares tq, so the
// per-token sequence data is wave-uniform: a wave whose windows all lie in
// one sequence takes a branch-free path, the others test token by token.
__device__ __forceinline__ float conv_tap4(const float4 wc, float bias, float h0, float h1,
                                           float h2, float x)
{
    float acc = bias;
    acc = fmaf(wc.x, h0, acc);
    acc = fmaf(wc.y, h1, acc);
    acc = fmaf(wc.z, h2, acc);
    acc = fmaf(wc.w, x, acc);
    return silu(acc);
}
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The 19 rows (clamped into [0, T)); issued early, consumed by conv_apply.
template <typename IOT>
__device__ __forceinline__ void conv_rows(float *xr, const PrefillArgs &a, int t0, int tq, int ch)
{
    // The window's rows t0 + tq - 3 .. t0 + tq + 15 (tq is the same in every
    // lane of a wave) through a buffer resource over its rows inside [0, T):
    // a row's address is one 32-bit add, and rows outside read as 0.
    // conv_apply never uses those: they lie before the sequence's first token
    // or past the input's end (tokens whose outputs are dropped).  A row
    // before the resource's first one has a negative offset, which as an
    // unsigned offset lies past the range.
    const int tb = __builtin_amdgcn_readfirstlane(t0 + tq - 3), b0 = max(tb, 0);
    const int rs = a.C * (int)sizeof(IOT);  // bytes between rows
    const int nrows = max(min(tb + 19, a.T) - b0, 0);
    const __amdgpu_buffer_rsrc_t xr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<IOT *>(static_cast<const IOT *>(a.x)) + (int64_t)b0 * a.C, (short)0, nrows * rs,
        0x00020000);
    const int vo = ch * (int)sizeof(IOT) + (tb - b0) * rs;
#pragma unroll
    for (int r = 0; r < 19; ++r) {
        if constexpr (sizeof(IOT) == 2)
            xr[r] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(xr_rsrc, vo + r * rs, 0, 0) << 16);
        else
            xr[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr_rsrc, vo + r * rs, 0, 0));
    }
}

// The conv weights and bias of channel ch.
__device__ __forceinline__ void conv_weights(float4 &wc, float &bias, const PrefillArgs &a, int ch)
{
    wc = reinterpret_cast<const float4 *>(a.w)[ch];
    bias = a.bias ? a.bias[ch] : 0.f;
}
__device__ __forceinline__ void conv_apply(float *y, const float *xr, const PrefillArgs &a, int t0,
                                           int tq, int ch, const int *sst, const int *ssl,
                                           float4 wc, float bias)
{
    const int s_first = wave_uniform(sst[tq]), s_last = wave_uniform(sst[tq + 15]);
    if (s_first == s_last && s_first <= t0 + tq - 3) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            y[i] = conv_tap4(wc, bias, xr[i], xr[i + 1], xr[i + 2], xr[i + 3]);
        return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tt = tq + i;
        const int nh = wave_uniform(sst[tt]) - (t0 + tt - 3);  // window rows before the start
        const int hrow = wave_uniform(ssl[tt]);
        float win[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) win[r] = r >= nh ? xr[i + r] : 0.f;
        if (nh > 0 && hrow >= 0) {
            const int64_t hb = (int64_t)hrow * a.conv_stride + ch;
#pragma unroll
            for (int r = 0; r < 3; ++r)
                if (r < nh) win[r] = load_elem(a.conv_pool, hb + (int64_t)(r + 3 - nh) * a.C,
                                               a.conv_dtype);
        }
        y[i] = conv_tap4(wc, bias, win[0], win[1], win[2], win[3]);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-block quantities, one workgroup (8 waves) per (tile, head).
// ---------------------------------------------------------------------------
constexpr int kIntraThreads = 512;
constexpr int kSeqTab = 512;  // sequences whose cu_seqlens / slot_in kernel 1 stages in LDS
static_assert(kSeqTab == kIntraThreads, "one table entry per thread");
constexpr size_t kIntraLdsFloats = 3 * kRegion + 2 * CB * LDJ + 2 * CB + 4 * DK;
constexpr size_t kIntraLds = kIntraLdsFloats * sizeof(float) + (5 * CB + 8 + 2 * kSeqTab) * sizeof(int);
// per-token flags of kernel 1 (sub-pieces)
enum { TF_OPEN = 1,      // no full reset between the piece start and the token
       TF_LAST = 2,      // no full reset after the token up to the piece end
       TF_PRESET = 4,    // the token's piece holds a full reset
       TF_RESET = 8 };   // the token itself resets every key channel

// Kernel 1 runs persistently: a grid of one workgroup per CU walks the
// (tile, head) items, item = tile * Hv + head.  The raw inputs phase 1 reads
// (thread (token t, 16-channel chunk c0): q, k, the gates and beta; with the
// fused conv the q and k conv windows and weights instead of q and k) are
// loaded for the next item while the current one runs, so an item starts on
// inputs already in registers.
template <typename IOT, bool KDA> struct IntraIn {
    static constexpr int QN = sizeof(IOT);  // 16-byte words per 16 q (or k) elements
    uint4 q[QN], k[QN];
    float4 g[KDA ? 4 : 1];
    float bt;
};
template <typename IOT, bool KDA>
__device__ __forceinline__ void intra_issue(IntraIn<IOT, KDA> &r, const PrefillArgs &a, int item,
                                            int t, int c0)
{
    const int tile = item / a.Hv, h = item - tile * a.Hv, kh = h / a.G;
    const int t0 = tile * CB, nt = min(CB, a.T - t0);
    const int64_t tok = t0 + min(t, nt - 1);
    if constexpr (KDA) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.g[i] = reinterpret_cast<const float4 *>(a.g + (tok * a.Hv + h) * DK + c0)[i];
    } else {
        r.g[0].x = a.g[tok * a.Hv + h];
    }
    r.bt = a.beta[tok * a.Hv + h];
    const uint4 *q = reinterpret_cast<const uint4 *>(static_cast<const IOT *>(a.q) + tok * a.q_stride + kh * DK + c0);
    const uint4 *k = reinterpret_cast<const uint4 *>(static_cast<const IOT *>(a.k) + tok * a.k_stride + kh * DK + c0);
#pragma unroll
    for (int i = 0; i < IntraIn<IOT, KDA>::QN; ++i) r.q[i] = q[i];
#pragma unroll
    for (int i = 0; i < IntraIn<IOT, KDA>::QN; ++i) r.k[i] = k[i];
}
template <typename IOT>
__device__ __forceinline__ void unpack16w(const uint4 *w, float *f)
{
#pragma unroll
    for (int i = 0; i < (int)sizeof(IOT); ++i) {
        const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(IOT) == 2) {
                f[8 * i + 2 * j] = bf16_lo(u[j]);
                f[8 * i + 2 * j + 1] = bf16_hi(u[j]);
            } else {
                f[4 * i + j] = __uint_as_float(u[j]);
            }
        }
    }
}
template <typename IOT, bool KDA>
__device__ __forceinline__ void intra_unpack(const IntraIn<IOT, KDA> &r, float *qv, float *kv,
                                             float *gv, float &bt)
{
    unpack16w<IOT>(r.q, qv);
    unpack16w<IOT>(r.k, kv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 g = r.g[KDA ? i : 0];
        gv[4 * i] = g.x;
        gv[4 * i + 1] = KDA ? g.y : g.x;
        gv[4 * i + 2] = KDA ? g.z : g.x;
        gv[4 * i + 3] = KDA ? g.w : g.x;
    }
    bt = r.bt;
}

// With the fused conv: the q and k channels' 19-row conv windows of thread
// (channel cc, tokens tc .. tc + 15), and the gates and beta of thread
// (token t, 16-channel chunk c0).
template <typename IOT, bool KDA> struct IntraConvIn {
    float xq[19], xk[19];
    float4 wq, wk;  // the two channels' conv weights and biases
    float bq, bk;
    float4 g[KDA ? 4 : 1];
    float bt;
};
template <typename IOT, bool KDA>
__device__ __forceinline__ void intra_issue_conv(IntraConvIn<IOT, KDA> &r, const PrefillArgs &a,
                                                 int item, int t, int c0, int cc, int tc)
{
    const int tile = item / a.Hv, h = item - tile * a.Hv, kh = h / a.G;
    const int t0 = tile * CB, nt = min(CB, a.T - t0);
    const int64_t tok = t0 + min(t, nt - 1);
    if constexpr (KDA) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.g[i] = reinterpret_cast<const float4 *>(a.g + (tok * a.Hv + h) * DK + c0)[i];
    } else {
        r.g[0].x = a.g[tok * a.Hv + h];
    }
    r.bt = a.beta[tok * a.Hv + h];
    conv_weights(r.wq, r.bq, a, kh * DK + cc);
    conv_weights(r.wk, r.bk, a, a.Hqk * DK + kh * DK + cc);
    conv_rows<IOT>(r.xq, a, t0, tc, kh * DK + cc);  // both windows in flight together
    conv_rows<IOT>(r.xk, a, t0, tc, a.Hqk * DK + kh * DK + cc);
}

// GDN with bf16 inputs in bf16x3 mode: the decayed queries are a per-token
// scale of the q rows, which are exact bf16 matrix-core operands, so kernel 1
// stores only that scale and the chain reads the q rows (shared by the value
// heads of a q/k head) instead of a split copy of Q Gamma.
template <typename IOT, bool KDA, int MODE, bool CONV> constexpr bool raw_q_chain()
{
    return !KDA && !CONV && MODE == PM_BF16X3 && std::is_same<IOT, bf16_t>::value;
}

template <typename IOT, bool KDA, int MODE, bool CONV>
__global__ void __launch_bounds__(kIntraThreads) prefill_intra_kernel(PrefillArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *Qn = sm;                  // q_hat [64][LDK]; later (beta K Gamma)^T [128][LDJ]
    float *Kn = Qn + kRegion;        // k_hat [64][LDK]; later (beta V)^T [128][LDJ]
    float *Gc = Kn + kRegion;        // cumulative log decay over the tile
    float *Nm = Gc + kRegion;        // N = Diag(beta) A (strictly lower, masked); earlier
                                     // K Gamma_L / Gamma (step 3)
    float *Tm = Nm + CB * LDJ;       // T = (I + N)^-1; in step 4 also a partial of A
    float *bet = Tm + CB * LDJ;      // beta
    float *qsum = bet + CB;          // [4][128] partial sums of the tile scan
    float *inq = qsum + 4 * DK;      // 1 / |q_t| (0 past the input's end)
    int *pst = reinterpret_cast<int *>(inq + CB);       // piece start, then sub-piece
                                                              // start (tile-local)
    int *pen = pst + CB;                                      // piece end (inclusive)
    int *sst = pen + CB;             // fused conv: the token's sequence start (global)
    int *ssl = sst + CB;             // fused conv: its history row (-1: zeros)
    int *bigw = ssl + CB;            // [8] KDA: wave w saw a sub-block span above kSpanMax
    int *tfl = bigw + 8;             // TF_* flags per token
    int *cut = tfl + CB;             // [kSeqTab] cu_seqlens (fewer than kSeqTab sequences)
    int *sit = cut + kSeqTab;        // [kSeqTab] slot_in
    float *XtK = Qn, *XtV = Kn;      // transposed right-hand sides of phase 6
    float *KhTl = Nm;                // [128][LDJ] staging of K Gamma_L / Gamma, transposed

    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    const int nitems = (a.T + CB - 1) / CB * a.Hv;
    // the store rounds of steps 3 and 5 run unrolled, so their loads and
    // exponentials overlap; with the fused conv's windows live that spills,
    // so there they stay loops
    constexpr int kStoreUnroll = CONV ? 1 : 4;
    constexpr bool kRawQ = raw_q_chain<IOT, KDA, MODE, CONV>();
    // With fewer than kSeqTab sequences, cu_seqlens and slot_in go to LDS
    // once (one entry per thread; entries past N repeat the last one and are
    // never read) and tokens search them there.  Larger batches search
    // cu_seqlens in global memory.
    const bool tab = a.N < kSeqTab;
    {
        const int i = threadIdx.x;
        cut[i] = a.cu[min(i, a.N)];
        sit[i] = a.slot_in[min(i, a.N - 1)];
    }
    __syncthreads();
    // The sequence of token t of an item (phase 1's mapping): its piece's
    // start and end in the tile, the sequence's first token, its slot_in row
    // (-1: none).  Found for the next item at the end of the current one's
    // step 1.
    struct Seq { int ps, pe, s0, hs; };
    auto find_seq_item = [&](int it, int t) {
        const int t0 = it / a.Hv * CB, nt = min(CB, a.T - t0);
        Seq r{t, t, 0, -1};
        if (t < nt) {
            int n, s0, s1, si;
            if (tab) {
                int lo = 0, hi = a.N - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (cut[mid] <= t0 + t) lo = mid;
                    else hi = mid - 1;
                }
                n = lo;
                s0 = cut[n];
                s1 = cut[n + 1];
                si = sit[n];
                // keeps these LDS reads from being merged with the global ones
                // below into one generic load, which would wait for every load
                asm volatile("" : "+v"(s0), "+v"(s1), "+v"(si));
            } else {
                n = find_seq_p(a.cu, a.N, t0 + t);
                s0 = a.cu[n];
                s1 = a.cu[n + 1];
                si = a.slot_in[n];
                // waits for these loads inside this branch, so the join
                // below does not wait for every memory operation in flight
                asm volatile("" : "+v"(s0), "+v"(s1), "+v"(si));
            }
            r.ps = max(s0, t0) - t0;
            r.pe = min(s1, t0 + CB) - 1 - t0;
            r.s0 = s0;
            r.hs = (si >= 0 && si < a.num_rows) ? si : -1;
        }
        return r;
    };
    // The items of workgroup w: i0 + k * stride, k < count.  Without the
    // fused conv a contiguous range, so consecutive items are the heads of
    // one tile, which share the sequence lookup (and, with GQA, the q/k
    // rows).  With it every gridDim.x-th item, so the heads of a tile run at
    // once on different CUs while their conv windows' rows sit in L2 (a
    // contiguous range was 1.8% slower there).
    const int G = gridDim.x, w = blockIdx.x;
    int i0, stride, count;
    if constexpr (CONV) {
        i0 = w;
        stride = G;
        count = (nitems - w + G - 1) / G;
    } else {
        const int per = nitems / G, rem = nitems % G;
        i0 = w * per + min(w, rem);
        stride = 1;
        count = per + (w < rem ? 1 : 0);
    }
    const int ilast = i0 + (count - 1) * stride;
    Seq nseq = find_seq_item(i0, threadIdx.x >> 3);
    // the next item's inputs: phase 1's mapping, and with the fused conv the
    // conv windows in its (channel, 16 tokens) mapping
    IntraIn<IOT, KDA> nx;
    IntraConvIn<IOT, KDA> ncx;
    if constexpr (CONV)
        intra_issue_conv(ncx, a, i0, threadIdx.x >> 3, 16 * (threadIdx.x & 7),
                         threadIdx.x & (DK - 1), 16 * (threadIdx.x >> 7));
    else
        intra_issue(nx, a, i0, threadIdx.x >> 3, 16 * (threadIdx.x & 7));
    // The first item waits for its loads here.  Later items find theirs
    // complete (see the end of step 1).  Without this wait the loop head
    // would merge the two cases and wait for every memory operation at each
    // item, including the previous item's last stores.
    __builtin_amdgcn_s_waitcnt(0);
    for (int item = i0; item <= ilast; item += stride) {
        // an opaque copy of the thread index per item: what derives from it
        // (lane offsets, LDS addresses) is formed inside the item and not
        // held live across the whole loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = tid >> 6;
        const int li = lane & 15, lq = lane >> 4;
        // phase 1's thread mapping: token t, 16-channel chunk cq
        const int t = tid >> 3, cq = tid & 7, c0 = 16 * cq;
        const int tile = item / a.Hv, h = item - tile * a.Hv, kh = h / a.G;
        const int t0 = tile * CB;
        const int nt = min(CB, a.T - t0);
        auto row = [&](int t) { return ((int64_t)(t0 + t) * a.Hv + h); };

        // ---- 1. inputs: thread (token t, 16-channel chunk cq), and the
        //         token's sequence found under the previous item
        const bool valid = t < nt;
        const Seq seq = nseq;
        const int ps = seq.ps, pe = seq.pe, s0 = seq.s0, hs = seq.hs;
        float qv[16], kv[16], gv[16], bt;
        // fused conv: thread (channel cc, 16 tokens tc .. tc + 15); every lane of
        // a wave shares tc, as conv_apply requires
        const int cc = tid & (DK - 1), tc = 16 * (tid >> 7);
        float xq[19], xk[19];
        if constexpr (CONV) {
#pragma unroll
            for (int r = 0; r < 19; ++r) {
                xq[r] = ncx.xq[r];
                xk[r] = ncx.xk[r];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 g = ncx.g[KDA ? i : 0];
                gv[4 * i] = g.x;
                gv[4 * i + 1] = KDA ? g.y : g.x;
                gv[4 * i + 2] = KDA ? g.z : g.x;
                gv[4 * i + 3] = KDA ? g.w : g.x;
            }
            bt = ncx.bt;
        } else {
            intra_unpack(nx, qv, kv, gv, bt);
        }
        // this item's LDS writes come after the previous item's last reads
        __syncthreads();
        if constexpr (CONV) {
            // conv of q and k into Qn / Kn, then back to the (token, chunk)
            // mapping for the norms
            if (cq == 0) {
                sst[t] = s0;
                ssl[t] = hs;
            }
            __syncthreads();
            float y[16];
            conv_apply(y, xq, a, t0, tc, kh * DK + cc, sst, ssl, ncx.wq, ncx.bq);
#pragma unroll
            for (int i = 0; i < 16; ++i) Qn[(tc + i) * LDK + cc] = y[i];
            conv_apply(y, xk, a, t0, tc, a.Hqk * DK + kh * DK + cc, sst, ssl, ncx.wk, ncx.bk);
#pragma unroll
            for (int i = 0; i < 16; ++i) Kn[(tc + i) * LDK + cc] = y[i];
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                const float4 q4 = *reinterpret_cast<const float4 *>(Qn + t * LDK + c0 + e);
                const float4 k4 = *reinterpret_cast<const float4 *>(Kn + t * LDK + c0 + e);
                qv[e] = q4.x; qv[e + 1] = q4.y; qv[e + 2] = q4.z; qv[e + 3] = q4.w;
                kv[e] = k4.x; kv[e + 1] = k4.y; kv[e + 2] = k4.z; kv[e + 3] = k4.w;
            }
        }
        float sq = 0.f, sk = 0.f, live = 0.f;  // live: channels not reset
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (!valid) { qv[e] = 0.f; kv[e] = 0.f; gv[e] = 0.f; }
            sq = fmaf(qv[e], qv[e], sq);
            sk = fmaf(kv[e], kv[e], sk);
            live += gv[e] > kGateFloor ? 1.f : 0.f;
        }
        sq = group_sum<8>(sq);
        sk = group_sum<8>(sk);
        live = group_sum<8>(live);
        const float iq = __builtin_amdgcn_rsqf(sq + a.eps), ik = __builtin_amdgcn_rsqf(sk + a.eps);
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            *reinterpret_cast<float4 *>(Qn + t * LDK + c0 + e) =
                make_float4(qv[e] * iq, qv[e + 1] * iq, qv[e + 2] * iq, qv[e + 3] * iq);
            *reinterpret_cast<float4 *>(Kn + t * LDK + c0 + e) =
                make_float4(kv[e] * ik, kv[e + 1] * ik, kv[e + 2] * ik, kv[e + 3] * ik);
            if (KDA || c0 == 0)  // GDN: one decay per token, kept in channel 0
                *reinterpret_cast<float4 *>(Gc + t * LDK + c0 + e) =
                    make_float4(fmaxf(gv[e], kGateFloor), fmaxf(gv[e + 1], kGateFloor),
                                fmaxf(gv[e + 2], kGateFloor), fmaxf(gv[e + 3], kGateFloor));
        }
        if (cq == 0) {
            bet[t] = valid ? bt : 0.f;
            inq[t] = valid ? iq : 0.f;
            pst[t] = ps;
            pen[t] = pe;
            tfl[t] = TF_OPEN | TF_LAST | (live == 0.f ? TF_RESET : 0);  // final unless a reset
        }
        // the next item's sequences and inputs (the last item repeats its
        // own, without a branch).  They are older than this item's v loads,
        // so step 6's wait for those completes them too, and the next item
        // starts without waiting.
        {
            const int next = min(item + stride, ilast);
            if (next / a.Hv != tile) nseq = find_seq_item(next, t);
            if constexpr (CONV) intra_issue_conv(ncx, a, next, t, c0, cc, tc);
            else intra_issue(nx, a, next, t, c0);
        }
        __syncthreads();
        // sub-pieces: with a full reset in the tile (rm, the same in every wave),
        // lane t of wave 0 finds the last reset at or before t and the last one
        // of its piece, then one more barrier publishes them
        const uint64_t rm = __ballot(tfl[lane] & TF_RESET);
        if (rm != 0 && wave == 0) {
            const bool rs = (rm >> lane) & 1;
            const int ps_l = pst[lane], pe_l = pen[lane];
            const uint64_t upto = rm & ((2ull << lane) - 1ull), upto_e = rm & ((2ull << pe_l) - 1ull);
            const int r = upto ? 63 - __builtin_clzll(upto) : -1;       // last reset <= t
            const int rl = upto_e ? 63 - __builtin_clzll(upto_e) : -1;  // last reset <= piece end
            pst[lane] = max(ps_l, r);
            tfl[lane] = (r < ps_l ? TF_OPEN : 0) | (rl <= lane ? TF_LAST : 0) |
                        (rl >= ps_l ? TF_PRESET : 0) | (rs ? TF_RESET : 0);
        }
        if (rm != 0) __syncthreads();

        // ---- 2. cumulative decay over the tile, segmented at piece starts: four
        //         quarters (the 16-token sub-blocks) of 16 tokens per channel.
        //         run is the sum inside the quarter since its last piece start;
        //         a quarter's tokens before its first sub-piece start continue the
        //         previous quarters' running sum.  -min(run) is the largest decay
        //         inside the sub-block, the span that bounds the factorised
        //         diagonal product of step 4.
        {
            const int c = tid & (DK - 1), qq = tid >> 7;
            // wave-uniform bit masks over the tile's tokens: sub-piece starts,
            // and full resets (those sub-pieces start from zero: the token's own
            // gate only empties what came before it)
            const uint64_t sm = __ballot(pst[lane] == lane);
            const uint32_t smq = (uint32_t)(sm >> (16 * qq)) & 0xFFFFu;
            const uint32_t rmq = (uint32_t)(rm >> (16 * qq)) & 0xFFFFu;
            const int first = smq ? __builtin_ctz(smq) : 16;  // first sub-piece start in the quarter
            const bool chan = KDA || c == 0;  // GDN: channel 0 only
            float run[16];
            float acc = 0.f, mn = 0.f;
            if (chan) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float gi = Gc[(16 * qq + i) * LDK + c];
                    acc = ((smq >> i) & 1) ? (((rmq >> i) & 1) ? 0.f : gi) : acc + gi;
                    run[i] = acc;
                    mn = fminf(mn, acc);
                }
                qsum[qq * DK + c] = acc;
            }
            if constexpr (KDA) {
                const bool big = __ballot(-mn > kSpanMax) != 0;
                if (lane == 0) bigw[wave] = big;
            }
            __syncthreads();
            // carry into the quarter: the running sum of the sub-piece open at
            // its start (quarter p restarts iff its last sub-piece began inside
            // it; quarter 0 always does, at the tile start)
            if (chan) {
                float off = 0.f;
                for (int p = 0; p < qq; ++p)
                    off = ((sm >> (16 * p)) & 0xFFFFu) ? qsum[p * DK + c] : off + qsum[p * DK + c];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    Gc[(16 * qq + i) * LDK + c] = i < first ? run[i] + off : run[i];
            }
        }
        __syncthreads();
        // GDN: one decay per token, so the decay factors of steps 3 and 6 are
        // per-token scalars, exp(G_end - G_t) and exp(G_t - G_start) over the
        // token's piece (zero across a reset), formed once here (qsum is free
        // after step 2)
        float *tabE = qsum, *tabS = qsum + CB;
        if constexpr (!KDA) {
            if (tid < CB) {
                const float G = Gc[tid * LDK];
                const int f = tfl[tid];
                tabE[tid] = (f & TF_LAST) ? exp_acc(Gc[pen[tid] * LDK] - G) : 0.f;
                tabS[tid] = (f & TF_OPEN) ? exp_acc(G) : 0.f;
            }
            __syncthreads();
        }

        // ---- 3. K Gamma_L / Gamma transposed through LDS and the piece's total
        //         decay (global, at piece ends): thread (token tt = lane, 16
        //         channels of wave w), so the transposed LDS writes of a wave run
        //         along the tokens and hit distinct banks; Q Gamma straight to
        //         global in fragment order
        const int64_t bh = (int64_t)tile * a.Hv + h;
        {
            const int tt = lane, c0 = 16 * wave;
            const int pen_t = pen[tt], f = tfl[tt];
            const bool last = f & TF_LAST, store_ge = tt < nt && tt == pen_t;
            float kh[16];
#pragma unroll
            for (int g4 = 0; g4 < 16; g4 += 4) {
                const float4 G = *reinterpret_cast<const float4 *>(Gc + tt * LDK + c0 + g4);
                // GDN keeps its decay in channel 0 only
                const float4 Ge = KDA ? *reinterpret_cast<const float4 *>(Gc + pen_t * LDK + c0 + g4)
                                      : make_float4(Gc[pen_t * LDK], Gc[pen_t * LDK], Gc[pen_t * LDK],
                                                    Gc[pen_t * LDK]);
                const float4 K = *reinterpret_cast<const float4 *>(Kn + tt * LDK + c0 + g4);
                if constexpr (KDA) {
                    // G_e <= G_t wherever the token is its piece's last (sums of
                    // gates <= 0 only fall), so the min changes nothing there and
                    // keeps the other lanes finite.  The exponentials are pinned
                    // as computed on every lane, so the masked products stay
                    // straight-line code.
                    const float e0 = exp_acc(fminf(Ge.x - G.x, 0.f)), e1 = exp_acc(fminf(Ge.y - G.y, 0.f));
                    const float e2 = exp_acc(fminf(Ge.z - G.z, 0.f)), e3 = exp_acc(fminf(Ge.w - G.w, 0.f));
                    asm volatile("" ::"v"(e0), "v"(e1), "v"(e2), "v"(e3));
                    kh[g4] = last ? K.x * e0 : 0.f;
                    kh[g4 + 1] = last ? K.y * e1 : 0.f;
                    kh[g4 + 2] = last ? K.z * e2 : 0.f;
                    kh[g4 + 3] = last ? K.w * e3 : 0.f;
                } else {
                    const float e = tabE[tt];
                    kh[g4] = K.x * e; kh[g4 + 1] = K.y * e; kh[g4 + 2] = K.z * e; kh[g4 + 3] = K.w * e;
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) KhTl[(c0 + i) * LDJ + tt] = kh[i];
            // the piece's decay of the state entering the tile (none left
            // after a full reset), stored by the piece's last token in one
            // branch after the straight-line products above
            if (store_ge) {
#pragma unroll
                for (int g4 = 0; g4 < 16; g4 += 4) {
                    const float4 Ge = KDA ? *reinterpret_cast<const float4 *>(Gc + pen_t * LDK + c0 + g4)
                                          : make_float4(Gc[pen_t * LDK], Gc[pen_t * LDK], Gc[pen_t * LDK],
                                                        Gc[pen_t * LDK]);
                    *reinterpret_cast<float4 *>(ws.Ge + row(tt) * DK + c0 + g4) =
                        (f & TF_PRESET) ? make_float4(kGateFloor, kGateFloor, kGateFloor, kGateFloor)
                                        : Ge;
                }
            }
        }
        if constexpr (MODE == PM_F32) {
#pragma unroll kStoreUnroll
            for (int rr = 0; rr < kBlkDK / 4 / kIntraThreads; ++rr) {
                const int idx = tid + rr * kIntraThreads;
                const int I = idx >> 9, g = (idx >> 6) & 7, ln = idx & 63;
                const int tt = 16 * I + (ln & 15), k0 = frag_off4<MODE, DK>(ln >> 4, g);
                const float4 qn = *reinterpret_cast<const float4 *>(Qn + tt * LDK + k0);
                float4 e4;
                if constexpr (KDA) {
                    const float4 G = *reinterpret_cast<const float4 *>(Gc + tt * LDK + k0);
                    const bool open = tfl[tt] & TF_OPEN;
                    e4 = make_float4(exp_if(open, G.x), exp_if(open, G.y), exp_if(open, G.z),
                                     exp_if(open, G.w));
                } else {
                    const float e = tabS[tt];
                    e4 = make_float4(e, e, e, e);
                }
                *reinterpret_cast<float4 *>(ws.Qt + bh * kBlkDK + 4 * idx) =
                    make_float4(qn.x * e4.x, qn.y * e4.y, qn.z * e4.z, qn.w * e4.w);
            }
        } else if constexpr (kRawQ) {
            // GDN, bf16 inputs: Q Gamma = Diag(s) Q with s_t = exp(G_t - G_start) / |q_t|,
            // so the chain reads the q rows themselves (exact bf16 operands) and s
            if (tid < CB) ws.Qt[bh * kBlkDK + tid] = inq[tid] * tabS[tid];
        } else {  // split layout: thread = (row block I, step m, lane), 8 channels
#pragma unroll kStoreUnroll
            for (int rr = 0; rr < kBlkDK / 8 / kIntraThreads; ++rr) {
                const int idx = tid + rr * kIntraThreads;
                const int I = idx >> 8, m = (idx >> 6) & 3, ln = idx & 63;
                const int tt = 16 * I + (ln & 15), k0 = 32 * m + 8 * (ln >> 4);
                const bool open = tfl[tt] & TF_OPEN;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = Qn[tt * LDK + k0 + e] *
                           (KDA ? exp_if(open, Gc[tt * LDK + k0 + e]) : tabS[tt]);
                store_split(ws.Qt + bh * kBlkDK + I * 2048, m, ln, v);
            }
        }
        __syncthreads();
        if constexpr (MODE == PM_F32) {
#pragma unroll kStoreUnroll
            for (int rr = 0; rr < kBlkDK / 4 / kIntraThreads; ++rr) {  // KhT in fragment order
                const int idx = tid + rr * kIntraThreads;
                const int cg = idx >> 8, g = (idx >> 6) & 3, ln = idx & 63;
                const int c = 16 * cg + (ln & 15), j0 = frag_off4<MODE, CB>(ln >> 4, g);
                *reinterpret_cast<float4 *>(ws.KhT + bh * kBlkDK + 4 * idx) =
                    *reinterpret_cast<const float4 *>(KhTl + c * LDJ + j0);
            }
        } else {
#pragma unroll kStoreUnroll
            for (int rr = 0; rr < kBlkDK / 8 / kIntraThreads; ++rr) {
                const int idx = tid + rr * kIntraThreads;
                const int cg = idx >> 7, m = (idx >> 6) & 1, ln = idx & 63;
                const int c = 16 * cg + (ln & 15), j0 = 32 * m + 8 * (ln >> 4);
                store_split(ws.KhT + bh * kBlkDK + cg * 1024, m, ln, KhTl + c * LDJ + j0);
            }
        }
        __syncthreads();
        // T's six upper tiles are cleared here and stay zero through steps 4 and
        // 5, which write only its lower tiles; every element of N is written by
        // step 4's mask pass
        if (tid < 6 * 64) {
            const int u = tid >> 6, r = (tid >> 2) & 15, q = tid & 3;  // tile (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
            const int I = u < 3 ? 0 : (u < 5 ? 1 : 2), J = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
            *reinterpret_cast<float4 *>(Tm + (16 * I + r) * LDJ + 16 * J + 4 * q) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        // the v loads of step 6 (its thread mapping: channel cc, tokens tc ..
        // tc + 15) run under steps 4 and 5: the 19-row conv window when the conv
        // is fused, else the 16 rows of v
        float xvr[19];
        if constexpr (CONV) {
            conv_rows<IOT>(xvr, a, t0, tc, 2 * a.Hqk * DK + h * DK + cc);
        } else {
            // through a buffer resource over the wave's rows tc .. nt - 1 of the
            // tile (tc is the same in every lane of a wave): a row's address is
            // one 32-bit add, and rows past the tile's end read as 0 (their
            // beta is 0 too)
            const int tw = __builtin_amdgcn_readfirstlane(tc);
            const int vs = (int)(a.v_stride * (int64_t)sizeof(IOT));  // bytes between rows
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<IOT *>(static_cast<const IOT *>(a.v)) + ((int64_t)(t0 + tw) * a.v_stride + h * DK),
                (short)0, max(nt - tw, 0) * vs, 0x00020000);
            const int vo = cc * (int)sizeof(IOT);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (sizeof(IOT) == 2)
                    xvr[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(vr, vo + i * vs, 0, 0) << 16);
                else
                    xvr[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, vo + i * vs, 0, 0));
            }
        }
        // (no barrier: step 4 reads neither N nor T until the barrier after
        // its row blocks, which orders the clearing above before its writes)

        // ---- 4. A and P.  Wave w contracts channel quarter qtr = w & 3 (32
        //         channels) for the block pairs of two row blocks: even waves
        //         take row block 3 (J = 0..3) and (0, 0), odd waves row blocks 2
        //         and 1; that is five pairs each.  A row block's left factors (its k and
        //         q rows decayed to the block's reference) are formed once for all
        //         its pairs.  Each pair is formed as the transposed tile, so lane
        //         (i, q) holds row 16I + i against columns 16J + 4q .. 16J + 4q + 3
        //         and every LDS access of the combining below is 16 bytes.  The
        //         four quarters' partial sums meet in LDS in a fixed order once Q
        //         is dead, so the result does not depend on which wave finishes
        //         first.
        constexpr int KQ = DK / 4, W = Step<MODE>::W, NS = KQ / Step<MODE>::K;
        const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform
        const int qtr = wv >> 1, grp = wv & 1;  // a quarter's two waves sit on different SIMDs
        f32x4 pa[5], pp[5];
        auto rowblock = [&](int I, int nJ, int k0) {
            const int ti = 16 * I + li;
            // the row's reference: G_{16I-1} if its piece began before the
            // sub-block, else 0 (the piece starts inside it)
            const bool cont = I > 0 && pst[ti] < 16 * I;
            // sub-block span above kSpanMax: the diagonal pair is formed per element
            const bool exact_diag =
                KDA && __builtin_amdgcn_readfirstlane(bigw[2 * I] | bigw[2 * I + 1]);
            float R[NS][W], fk[NS][W], fq[NS][W], fd[NS][W];
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    const int c = qtr * KQ + frag_k<MODE, KQ>(lq, st * W + e);
                    if constexpr (KDA) {
                        R[st][e] = I ? Gc[(16 * I - 1) * LDK + c] : 0.f;
                        const float x = Gc[ti * LDK + c] - (cont ? R[st][e] : 0.f);  // <= 0
                        const float et = exp_acc(fminf(x, kExpClamp));
                        fk[st][e] = Kn[ti * LDK + c] * et;
                        fq[st][e] = Qn[ti * LDK + c] * et;
                        // the diagonal's j-side factor (its column token is
                        // this row), e^-x as the reciprocal of e^x: it is read
                        // only when the sub-block's span is at most kSpanMax,
                        // where x >= -kSpanMax (flagged blocks take the
                        // per-element path below)
                        fd[st][e] = Kn[ti * LDK + c] * __builtin_amdgcn_rcpf(et);
                    } else {  // GDN: plain k and q rows; the decay is applied per element below
                        fk[st][e] = Kn[ti * LDK + c];
                        fq[st][e] = Qn[ti * LDK + c];
                        fd[st][e] = fk[st][e];
                    }
                }
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J >= nJ) break;
                const int tj = 16 * J + li;
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
                if (J == I && exact_diag) {
                    // exp(G_t - G_j) per element, t = ti, j = 16J + 4 lq + r: the
                    // transposed tile layout of the matrix-core path; pairs of
                    // other pieces or with j > t are masked later and only kept
                    // finite
#pragma unroll 2
                    for (int c = qtr * KQ; c < qtr * KQ + KQ; c += 4) {
                        const float4 kt = *reinterpret_cast<const float4 *>(Kn + ti * LDK + c);
                        const float4 qt = *reinterpret_cast<const float4 *>(Qn + ti * LDK + c);
                        const float4 gt = *reinterpret_cast<const float4 *>(Gc + ti * LDK + c);
                        const float ktv[4] = {kt.x, kt.y, kt.z, kt.w};
                        const float qtv[4] = {qt.x, qt.y, qt.z, qt.w};
                        const float gtv[4] = {gt.x, gt.y, gt.z, gt.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int jr = 16 * J + 4 * lq + r;
                            const float4 kj = *reinterpret_cast<const float4 *>(Kn + jr * LDK + c);
                            const float4 gj = *reinterpret_cast<const float4 *>(Gc + jr * LDK + c);
                            const float kjv[4] = {kj.x, kj.y, kj.z, kj.w}, gjv[4] = {gj.x, gj.y, gj.z, gj.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float kd = kjv[e] * exp_acc(fminf(gtv[e] - gjv[e], 0.f));
                                accA[r] = fmaf(ktv[e], kd, accA[r]);
                                accP[r] = fmaf(qtv[e], kd, accP[r]);
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        float fj[W];
#pragma unroll
                        for (int e = 0; e < W; ++e) {
                            const int c = qtr * KQ + frag_k<MODE, KQ>(lq, st * W + e);
                            fj[e] = J == I ? fd[st][e]
                                  : KDA ? Kn[tj * LDK + c] * exp_acc(fminf(R[st][e] - Gc[tj * LDK + c], kExpClamp))
                                        : Kn[tj * LDK + c];
                        }
                        mma_step_t<MODE>(accA, fk[st], fj);
                        mma_step_t<MODE>(accP, fq[st], fj);
                    }
                }
                pa[k0 + J] = accA;
                pp[k0 + J] = accP;
            }
        };
        if (grp == 0) {
            rowblock(3, 4, 0);
            rowblock(0, 1, 4);
        } else {
            rowblock(2, 3, 0);
            rowblock(1, 2, 3);
        }
        // the wave's pairs in the order of pa / pp: (3,0..3), (0,0) for group 0;
        // (2,0..2), (1,0..1) for group 1
        auto pairI = [&](int k) { return grp ? (k < 3 ? 2 : 1) : (k < 4 ? 3 : 0); };
        auto pairJ = [&](int k) { return grp ? (k < 3 ? k : k - 3) : (k < 4 ? k : 0); };
        __syncthreads();
        float *Ps = Qn;            // P [64][LDJ]; q_hat is no longer read
        float *Ps2 = Qn + CB * LDJ;  // second half of Q's space: P partial of quarters 2 + 3
        float *Nm2 = Tm;           // A partial of quarters 2 + 3 (T's lower tiles, rewritten in step 5)
        // The quarters' partial sums meet in a fixed order, (q0 + q1) + (q2 + q3):
        // quarters 0 and 2 store theirs, quarters 1 and 3 add theirs in place,
        // then every thread combines the two halves of its elements.
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if ((qtr & 1) == st) {
                float *dA = qtr < 2 ? Nm : Nm2, *dP = qtr < 2 ? Ps : Ps2;
                f32x4 prevA[5], prevP[5];
#pragma unroll
                for (int k = 0; k < 5; ++k) {
                    const int at = (16 * pairI(k) + li) * LDJ + 16 * pairJ(k) + 4 * lq;
                    prevA[k] = st ? *reinterpret_cast<const f32x4 *>(dA + at) : f32x4{0.f, 0.f, 0.f, 0.f};
                    prevP[k] = st ? *reinterpret_cast<const f32x4 *>(dP + at) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int k = 0; k < 5; ++k) {
                    const int at = (16 * pairI(k) + li) * LDJ + 16 * pairJ(k) + 4 * lq;
                    *reinterpret_cast<f32x4 *>(dA + at) = st ? prevA[k] + pa[k] : pa[k];
                    *reinterpret_cast<f32x4 *>(dP + at) = st ? prevP[k] + pp[k] : pp[k];
                }
            }
            __syncthreads();
        }
        // A keeps beta[t] A where j < t in the same piece (else 0), P keeps
        // j <= t in the same piece (GDN: also the element's decay
        // exp(G_t - G_j), <= 1 where it is kept); upper tiles are zero.  Thread
        // (row tt, columns j0 .. j0 + 3), straight-line: the upper tiles' sums
        // (zeros in A, stale rows in P) are read and then discarded by the masks.
        static_assert(CB * CB / 4 % kIntraThreads == 0, "whole mask rounds");
#pragma unroll
        for (int rr = 0; rr < CB * CB / 4 / kIntraThreads; ++rr) {
            const int idx = tid + rr * kIntraThreads;
            const int tt = idx >> 4, j0 = 4 * (idx & 15), at = tt * LDJ + j0;
            const f32x4 av = *reinterpret_cast<const f32x4 *>(Nm + at) + *reinterpret_cast<const f32x4 *>(Nm2 + at);
            const f32x4 pv = *reinterpret_cast<const f32x4 *>(Ps + at) + *reinterpret_cast<const f32x4 *>(Ps2 + at);
            const int p0 = pst[tt];
            const float bt = bet[tt];
            f32x4 na, np;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                float a1 = av[q], p1 = pv[q];
                if constexpr (!KDA) {
                    const float e = exp_acc(fminf(Gc[tt * LDK] - Gc[j * LDK], 0.f));
                    a1 *= e;
                    p1 *= e;
                }
                const bool same = j >= p0 && tt < nt;
                na[q] = same && j < tt ? bt * a1 : 0.f;
                np[q] = same && j <= tt ? p1 : 0.f;
            }
            *reinterpret_cast<f32x4 *>(Nm + at) = na;
            *reinterpret_cast<f32x4 *>(Ps + at) = np;
        }
        __syncthreads();

        // ---- 5. T = (I + N)^-1: diagonal 16x16 blocks by forward substitution
        //         (waves 0..3, lane c < 16 holds column c), then the off-diagonal
        //         blocks level by level: T_IJ = -T_II sum_{K=J}^{I-1} N_IK T_KJ.
        //         Meanwhile waves 4..7 store P and form step 6's (beta K Gamma)^T
        //         before the barrier that ends the diagonal solve, and write it to
        //         Q's space after that barrier, once P's store has freed it.
        if (wave < 4) {
            if (lane < 16) {
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
        }
        // step 6's (beta K Gamma)^T, formed by waves 4..7 before the barrier that
        // ends the diagonal solve and written to Q's space after it: thread
        // (rows 4 rq .. 4 rq + 3, tokens 8 tg .. 8 tg + 7).  In bf16x3 mode row
        // rho holds channel pi(rho), bits 2 and 3 of the index swapped (pi is its
        // own inverse): the row order in which step 7's transposed W product
        // reads it without bank conflicts.  pi keeps bits 0 and 1, so a thread's
        // four rows are four consecutive channels, read 16 bytes at a time.
        const int xu = tid - 256, rq = xu & 31, tg = xu >> 5;
        const int xc = MODE == PM_F32 ? 4 * rq : (4 * rq & ~12) | ((4 * rq & 4) << 1) | ((4 * rq & 8) >> 1);
        float bk[8][4];  // [token][row]
        auto form_bk = [&](int i) {
            const int tt = 8 * tg + i;
            const float4 K4 = *reinterpret_cast<const float4 *>(Kn + tt * LDK + xc);
            const float kv[4] = {K4.x, K4.y, K4.z, K4.w};
            if constexpr (KDA) {
                const float4 G4 = *reinterpret_cast<const float4 *>(Gc + tt * LDK + xc);
                const float gv[4] = {G4.x, G4.y, G4.z, G4.w};
                const bool open = tfl[tt] & TF_OPEN;
                const float b = bet[tt];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = b * kv[r] * exp_if(open, gv[r]);
                    bk[i][r] = open ? x : 0.f;
                }
            } else {
                const float b = bet[tt], e = tabS[tt];
#pragma unroll
                for (int r = 0; r < 4; ++r) bk[i][r] = b * kv[r] * e;
            }
        };
        constexpr int kPre = CONV && KDA ? 4 : 8;
        if (wave >= 4) {  // P to global in fragment order
            if constexpr (MODE == PM_F32) {
#pragma unroll kStoreUnroll
                for (int rr = 0; rr < kBlkCB / 4 / 256; ++rr) {
                    const int idx = tid - 256 + rr * 256;
                    const int I = idx >> 8, g = (idx >> 6) & 3, ln = idx & 63;
                    const int tt = 16 * I + (ln & 15), j0 = frag_off4<MODE, CB>(ln >> 4, g);
                    *reinterpret_cast<float4 *>(ws.P + bh * kBlkCB + 4 * idx) =
                        *reinterpret_cast<const float4 *>(Ps + tt * LDJ + j0);
                }
            } else {
#pragma unroll kStoreUnroll
                for (int rr = 0; rr < kBlkCB / 8 / 256; ++rr) {
                    const int idx = tid - 256 + rr * 256;
                    const int I = idx >> 7, m = (idx >> 6) & 1, ln = idx & 63;
                    const int tt = 16 * I + (ln & 15), j0 = 32 * m + 8 * (ln >> 4);
                    store_split(ws.P + bh * kBlkCB + I * 1024, m, ln, Ps + tt * LDJ + j0);
                }
            }
            // (beta K Gamma)^T under the diagonal solve (with the fused conv's
            // windows live, half of it, to stay within the registers)
#pragma unroll
            for (int i = 0; i < kPre; ++i) form_bk(i);
        }
        __syncthreads();  // diagonal blocks of T done; P is read out
        if (wave >= 4) {
#pragma unroll
            for (int i = kPre; i < 8; ++i) form_bk(i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *row = XtK + (4 * rq + r) * LDJ;
                const float v[8] = {bk[0][r], bk[1][r], bk[2][r], bk[3][r], bk[4][r], bk[5][r], bk[6][r], bk[7][r]};
                if constexpr (MODE == PM_F32) {
                    *reinterpret_cast<float4 *>(row + 8 * tg) = make_float4(v[0], v[1], v[2], v[3]);
                    *reinterpret_cast<float4 *>(row + 8 * tg + 4) = make_float4(v[4], v[5], v[6], v[7]);
                } else {  // split row: hi words 0..31, lo words 32..63 for tokens 0..63
                    uint4 hi, lo;
                    split8(v, hi, lo);
                    *reinterpret_cast<uint4 *>(row + 4 * tg) = hi;
                    *reinterpret_cast<uint4 *>(row + 32 + 4 * tg) = lo;
                }
            }
        }
        // Column block J of T depends only on its own earlier blocks and on
        // the diagonal blocks, so wave J (< 3) walks I = J + 1 .. 3 alone, and
        // one barrier closes the step.  Its products take the contraction index
        // of step s in lane quad q as k = 4q + s: lane (i, q) then supplies row i
        // of the left factor (one 16-byte read of N or T_II) and holds, in its
        // result registers, exactly the right factor of the next product (X for
        // T_II X, and T_IJ for the later X's), so the chain stays in registers.
        auto levels = [&](auto Jc) {
            constexpr int J = decltype(Jc)::value;
            f32x4 Tc[4];  // Tc[K][s] = T_KJ[4 lq + s][li]
#pragma unroll
            for (int s = 0; s < 4; ++s) Tc[J][s] = Tm[(16 * J + 4 * lq + s) * LDJ + 16 * J + li];
#pragma unroll
            for (int I = J + 1; I < 4; ++I) {
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = J; K < I; ++K) {
                    const f32x4 n4 = *reinterpret_cast<const f32x4 *>(Nm + (16 * I + li) * LDJ + 16 * K + 4 * lq);
#pragma unroll
                    for (int s = 0; s < 4; ++s) X = mfma4(n4[s], Tc[K][s], X);
                }
                const f32x4 t4 = *reinterpret_cast<const f32x4 *>(Tm + (16 * I + li) * LDJ + 16 * I + 4 * lq);
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) Y = mfma4(t4[s], X[s], Y);
                Tc[I] = -Y;
#pragma unroll
                for (int r = 0; r < 4; ++r) Tm[(16 * I + 4 * lq + r) * LDJ + 16 * J + li] = -Y[r];
            }
        };
        if (wv == 0) levels(std::integral_constant<int, 0>{});
        else if (wv == 1) levels(std::integral_constant<int, 1>{});
        else if (wv == 2) levels(std::integral_constant<int, 2>{});
        __syncthreads();

        // ---- 6. right-hand sides, transposed: (beta V)^T here, (beta K Gamma)^T
        //         formed under step 5.  In bf16x3 mode they and T are stored
        //         split (bf16 hi / lo rows), so step 7 reads its operands without
        //         converting them; T goes to N's space, which is dead.
        if constexpr (MODE != PM_F32) {
            const int row = tid >> 3, k0 = 8 * (tid & 7);
            const float4 t0v = *reinterpret_cast<const float4 *>(Tm + row * LDJ + k0);
            const float4 t1v = *reinterpret_cast<const float4 *>(Tm + row * LDJ + k0 + 4);
            const float tv[8] = {t0v.x, t0v.y, t0v.z, t0v.w, t1v.x, t1v.y, t1v.z, t1v.w};
            uint4 hi, lo;
            split8(tv, hi, lo);
            *reinterpret_cast<uint4 *>(Nm + row * LDJ + k0 / 2) = hi;
            *reinterpret_cast<uint4 *>(Nm + row * LDJ + 32 + k0 / 2) = lo;
        }
        {   // thread (channel c, 16 tokens): rows of (beta V)^T, loads coalesced over c
            const int c = tid & (DK - 1), tq = 16 * (tid >> 7);
            float xv[16];
            if constexpr (CONV) {  // c, tq are cc, tc
                float4 wv;
                float bv;
                conv_weights(wv, bv, a, 2 * a.Hqk * DK + h * DK + c);
                conv_apply(xv, xvr, a, t0, tq, 2 * a.Hqk * DK + h * DK + c, sst, ssl, wv, bv);
#pragma unroll
                for (int i = 0; i < 16; ++i) xv[i] *= bet[tq + i];  // bet = 0 past nt
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xv[i] = bet[tq + i] * xvr[i];  // bet = 0 past nt
            }
            // K's space is free: its last reads formed (beta K Gamma)^T under step 5
            if constexpr (MODE == PM_F32) {
#pragma unroll
                for (int i = 0; i < 16; i += 4)
                    *reinterpret_cast<float4 *>(XtV + c * LDJ + tq + i) =
                        make_float4(xv[i], xv[i + 1], xv[i + 2], xv[i + 3]);
            } else {
                store_row_split16(XtV + c * LDJ, tq, xv);
            }
        }
        __syncthreads();

        // ---- 7. U = T (beta V) and W = T (beta K Gamma).  U: wave w owns
        //         output columns 16w .. 16w + 15 for the four token blocks and
        //         leaves them in the result layout.  W, fp32 mode: the same, staged
        //         in LDS (the decay cumsum is dead) and stored in fragment order.
        //         W, bf16x3 mode: wave w takes the 32-channel step s = w & 3 of
        //         token blocks w >> 2 and 3 - (w >> 2) and forms W^T tiles whose
        //         rows are channels 32 s + 8 (i >> 2) + 4 h + (i & 3), h = 0, 1: each
        //         lane then holds the 8 consecutive channels of one token that W's
        //         fragment order wants, and stores them split from registers.
        float *Wst = Gc;  // [64][LDK]
        {
            const int C = wave;
#pragma unroll
            for (int which = 0; which < (MODE == PM_F32 ? 2 : 1); ++which) {
                const float *Xt = which ? XtK : XtV;
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (MODE == PM_F32) {
                        const float *Trow = Tm + (16 * I + li) * LDJ, *Xrow = Xt + (16 * C + li) * LDJ;
                        auto fa = [&](int, int j) { return Trow[j]; };
                        auto fb = [&](int, int j) { return Xrow[j]; };
                        if (I < 2) mma_gen<MODE, 32>(acc, lq, fa, fb);  // T rows < 32: columns < 32
                        else mma_gen<MODE, 64>(acc, lq, fa, fb);
                    } else {  // split rows: step m, lane quad lq covers columns 32 m + 8 lq ..
                        const float *Trow = Nm + (16 * I + li) * LDJ, *Xrow = Xt + (16 * C + li) * LDJ;
#pragma unroll
                        for (int m = 0; m < (I < 2 ? 1 : 2); ++m) {
                            const int o = 16 * m + 4 * lq;
                            const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(Trow + o);
                            const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(Trow + 32 + o);
                            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(Xrow + o);
                            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(Xrow + 32 + o);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
                        }
                    }
                    if (which == 0) {
                        *reinterpret_cast<f32x4 *>(ws.U + bh * kBlkDK + fidx(I * 8 + C, lane)) = acc;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) Wst[(16 * I + 4 * lq + r) * LDK + 16 * C + li] = acc[r];
                    }
                }
            }
        }
        if constexpr (MODE == PM_F32) {
            __syncthreads();
            // fixed trip counts, unrolled (the thread index is opaque here, so a
            // strided loop would not be)
#pragma unroll
            for (int r = 0; r < kBlkDK / 4 / kIntraThreads; ++r) {
                const int idx = tid + r * kIntraThreads;
                const int I = idx >> 9, g = (idx >> 6) & 7, ln = idx & 63;
                const int tt = 16 * I + (ln & 15), k0 = frag_off4<MODE, DK>(ln >> 4, g);
                *reinterpret_cast<float4 *>(ws.W + bh * kBlkDK + 4 * idx) =
                    *reinterpret_cast<const float4 *>(Wst + tt * LDK + k0);
            }
        } else {
            const int st = wv & 3;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int I = k ? 3 - (wv >> 2) : wv >> 2;
                const float *Trow = Nm + (16 * I + li) * LDJ;
                float v[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    // channel 32 st + 8 (li >> 2) + 4 hh + (li & 3) sits in row pi of it
                    const float *Xrow = XtK + (32 * st + 16 * (li >> 3) + 8 * hh + (li & 7)) * LDJ;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        if (m == 1 && I < 2) break;  // T rows < 32: columns < 32
                        const int o = 16 * m + 4 * lq;
                        const bf16x8_t xh = *reinterpret_cast<const bf16x8_t *>(Xrow + o);
                        const bf16x8_t xl = *reinterpret_cast<const bf16x8_t *>(Xrow + 32 + o);
                        const bf16x8_t th = *reinterpret_cast<const bf16x8_t *>(Trow + o);
                        const bf16x8_t tl = *reinterpret_cast<const bf16x8_t *>(Trow + 32 + o);
                        // the three products in the order U's take them: lo(T) hi(X),
                        // hi(T) lo(X), hi(T) hi(X)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, tl, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, th, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, th, acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[4 * hh + r] = acc[r];
                }
                store_split(ws.W + bh * kBlkDK + I * 2048, st, lane, v);
            }
        }
    }
}

// Chain workgroups: S row slices of each (sequence, head) pair, launched as a
// 1-D grid of ceil(N Hv / 8) * 8 S workgroups.  Workgroup L takes pair
// 8 (L / 8S) + L % 8 and slice (L / 8) % S, so the slices of a pair are 8 ids
// apart: workgroups go to the 8 XCDs round-robin, so these share an XCD and
// run at about the same time, and the block operands they all read come from
// that XCD's L2 after the first.  Returns false for the padding workgroups.
__device__ __forceinline__ bool chain_ids(const PrefillArgs &a, int S, int &n, int &h, int &rs)
{
    const int L = blockIdx.x;
    const int pair = 8 * (L / (8 * S)) + (L & 7);
    rs = (L >> 3) % S;
    if (pair >= a.N * a.Hv) return false;
    n = pair / a.Hv;
    h = pair % a.Hv;
    return true;
}
inline unsigned chain_grid(const PrefillArgs &a, int S)
{
    return (unsigned)(((int64_t)a.N * a.Hv + 7) / 8 * 8 * S);
}

// ---------------------------------------------------------------------------
// Kernel 2: the block chain, one workgroup per (sequence, head, 16 state rows).
// Waves 0..3 ("row waves") own token rows 16I.. of D and O; waves 4..7
// ("column waves") own state columns 32(w-4) .. 32(w-4) + 31 of the update.
// All of a tile's operands are loaded into registers while the previous tile
// computes (ping-pong buffers), and the state slice is double-buffered in LDS,
// so a tile costs two barriers: D, then the output and the new state side by
// side.
// ---------------------------------------------------------------------------
constexpr int kChainThreads = 512;
constexpr size_t kChainLds = (2 * 16 * LDK + 16 * LDJ) * sizeof(float);

// Per-lane operands of one tile.  Row waves: [0, 32) W row fragment (K = 128
// channels), [32, 36) U in the result layout, [36, 68) Q Gamma row fragment,
// [68, 84) P row fragment (K = 64 tile-local tokens).  Column waves: [0, 32)
// K^T row fragments of two column tiles (K = 64 tokens), [32, 34) Gamma_L of
// the lane's two columns.  The two roles run separate loops with the same
// barrier sequence, so each keeps its own arrays in registers.
constexpr int kRowOps = 84, kColOps = 34;

template <typename IOT, typename ST, int MODE>
__global__ void __launch_bounds__(kChainThreads) prefill_chain_kernel(PrefillArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *Sbuf = sm;                 // two state slices [16 rows][LDK]
    float *Dt = sm + 2 * 16 * LDK;    // D^T of the tile [16 rows][LDJ] (tile-local tokens)

    int n, h, rs;  // rows 16 rs .. 16 rs + 15
    if (!chain_ids(a, DK / 16, n, h, rs)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
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
        Sbuf[i * LDK + c] = v;
    }

    const int tb0 = start / CB, tb1 = end > start ? (end - 1) / CB : tb0 - 1;
    const int ntiles = tb1 - tb0 + 1;  // 0 for an empty sequence
    // Both roles run the same barrier sequence: two per block.  The block loop
    // is unrolled by two over a pair of operand buffers (ping-pong), so the
    // loads for block it + 1, issued as block it starts, are first waited for
    // when block it + 1 computes.  Full 64-token blocks (the common case) skip
    // the piece masks.
    if (wave < 4) {
        auto load_ops = [&](int tb, float *ops) {
            const int64_t bh = (int64_t)tb * a.Hv + h;
            load_run(ops, ws.W + bh * kBlkDK + fidx(8 * I, 0), 8, lane);
            load_run(ops + 32, ws.U + bh * kBlkDK + fidx(8 * I + rs, 0), 1, lane);
            load_run(ops + 36, ws.Qt + bh * kBlkDK + fidx(8 * I, 0), 8, lane);
            load_run(ops + 68, ws.P + bh * kBlkCB + fidx(4 * I, 0), 4, lane);
        };
        auto block = [&](int it, const float *cur) {
            const int tb = tb0 + it, base = tb * CB;
            const int p0 = max(start, base) - base, p1 = min(end, base + CB) - base;
            const bool full = p0 == 0 && p1 == CB;
            __syncthreads();  // state slice in place, last D^T consumed
            const float *Srow = Sbuf + (it & 1) * 16 * LDK + li * LDK, *Drow = Dt + li * LDJ;
            auto lds_s = [&](int, int c) { return Srow[c]; };
            // D = U - W S^T, rows outside the piece masked
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (full) {
                mma_gen<MODE, DK>(acc, lq, [&](int idx, int) { return cur[idx]; }, lds_s);
            } else {
                const int ti = 16 * I + li;
                const bool in_i = ti >= p0 && ti < p1;
                mma_gen<MODE, DK>(acc, lq, [&](int idx, int) { return in_i ? cur[idx] : 0.f; },
                                  lds_s);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * I + 4 * lq + r;
                const bool in_r = tr >= p0 && tr < p1;
                Dt[li * LDJ + tr] = in_r ? cur[32 + r] - acc[r] : 0.f;
            }
            __syncthreads();  // D^T complete
            // O = scale (Q Gamma S^T + P D)
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            mma_gen<MODE, DK>(acc, lq, [&](int idx, int) { return cur[36 + idx]; }, lds_s);
            mma_gen<MODE, CB>(acc, lq, [&](int idx, int) { return cur[68 + idx]; },
                              [&](int, int j) { return Drow[j]; });
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tr = 16 * I + 4 * lq + r;
                if (tr >= p0 && tr < p1)
                    st<IOT>(a.out, ((int64_t)(base + tr) * a.Hv + h) * DK + 16 * rs + li,
                            a.scale * acc[r]);
            }
        };
        float bufA[kRowOps], bufB[kRowOps];
        if (ntiles > 0) load_ops(tb0, bufA);
        for (int it = 0; it < ntiles; it += 2) {
            load_ops(min(tb0 + it + 1, tb1), bufB);
            block(it, bufA);
            if (it + 1 >= ntiles) break;
            load_ops(min(tb0 + it + 2, tb1), bufA);
            block(it + 1, bufB);
        }
    } else {
        auto load_ops = [&](int tb, float *ops) {
            const int pend = min(end, tb * CB + CB) - 1;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = 32 * I + 16 * q + li;
                load_run(ops + 16 * q,
                         ws.KhT + ((int64_t)tb * a.Hv + h) * kBlkDK + fidx(4 * (2 * I + q), 0), 4,
                         lane);
                ops[32 + q] = ws.Ge[((int64_t)pend * a.Hv + h) * DK + c];
            }
        };
        auto block = [&](int it, const float *cur) {
            const int tb = tb0 + it, base = tb * CB;
            const int p0 = max(start, base) - base, p1 = min(end, base + CB) - base;
            const bool full = p0 == 0 && p1 == CB;
            const float *Scur = Sbuf + (it & 1) * 16 * LDK;
            float *Snext = Sbuf + ((it & 1) ^ 1) * 16 * LDK;
            const float *Drow = Dt + li * LDJ;
            __syncthreads();
            float sc[2][4];  // this lane's old state entries, read while D is formed
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sc[q][r] = Scur[(4 * lq + r) * LDK + 32 * I + 16 * q + li];
            __syncthreads();  // D^T complete
            // new state columns: S Gamma_L + D^T K^  (K^ columns outside the piece masked)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (full) {
                    mma_gen<MODE, CB>(acc, lq, [&](int, int j) { return Drow[j]; },
                                      [&](int idx, int) { return cur[16 * q + idx]; });
                } else {
                    mma_gen<MODE, CB>(acc, lq, [&](int, int j) { return Drow[j]; },
                                      [&](int idx, int j) {
                                          return (j >= p0 && j < p1) ? cur[16 * q + idx] : 0.f;
                                      });
                }
                const int c = 32 * I + 16 * q + li;
                const float gm = exp_acc(cur[32 + q]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Snext[(4 * lq + r) * LDK + c] = fmaf(sc[q][r], gm, acc[r]);
            }
        };
        float bufA[kColOps], bufB[kColOps];
        if (ntiles > 0) load_ops(tb0, bufA);
        for (int it = 0; it < ntiles; it += 2) {
            load_ops(min(tb0 + it + 1, tb1), bufB);
            block(it, bufA);
            if (it + 1 >= ntiles) break;
            load_ops(min(tb0 + it + 2, tb1), bufA);
            block(it + 1, bufB);
        }
    }
    __syncthreads();
    const float *Sfin = Sbuf + (ntiles & 1) * 16 * LDK;
    for (int idx = tid; idx < 16 * DK; idx += kChainThreads) {
        const int i = idx / DK, c = idx % DK;
        st<ST>(a.ssm_pool, (int64_t)so * a.ssm_stride + ((int64_t)h * DK + 16 * rs + i) * DK + c,
               Sfin[i * LDK + c]);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2, bf16x3 mode: the same chain with every matrix-core operand already
// split into bf16 hi / lo.  The workspace holds W, Q Gamma, P and the
// transposed decayed keys split (hi quad in run 2m, lo quad in run 2m + 1 for
// step m); the state slice is kept in LDS both in fp32 (for the update) and
// split, and D^T only split.  A 32-deep step is then two 16-byte reads or
// register quads per operand and three v_mfma_f32_16x16x32_bf16.  Tokens
// outside the piece need no operand masks: their D rows are stored as zeros
// and every other operand there is finite.
// ---------------------------------------------------------------------------
constexpr int LDKH = DK + 8;   // bf16 row stride of the split state (272 B = 4 mod 32 words)
constexpr int LDJH = CB + 8;   // bf16 row stride of the split D^T (144 B)

__device__ __forceinline__ bf16x8_t quad8(const float *w)
{
    return __builtin_bit_cast(bf16x8_t, make_uint4(__float_as_uint(w[0]), __float_as_uint(w[1]),
                                                   __float_as_uint(w[2]), __float_as_uint(w[3])));
}
__device__ __forceinline__ bf16x8_t lds8(const bf16_t *p)
{
    return *reinterpret_cast<const bf16x8_t *>(p);
}
__device__ __forceinline__ void mma3(f32x4 &acc, bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}
__device__ __forceinline__ void split1(float v, bf16_t &hi, bf16_t &lo)
{
    hi = f32_to_bf16(v);
    lo = f32_to_bf16(v - bf16_to_f32(hi));
}
// The same for two values at once: one packed conversion per part, the hi
// values read back from the packed dword (equal to split1 of each value).
__device__ __forceinline__ void split2(float v0, float v1, bf16_t &h0, bf16_t &h1, bf16_t &l0,
                                       bf16_t &l1)
{
    const uint32_t h = pack_bf16x2(v0, v1);
    const uint32_t l = pack_bf16x2(v0 - __uint_as_float(h << 16), v1 - __uint_as_float(h & 0xFFFF0000u));
    h0 = (bf16_t)(h & 0xFFFFu);
    h1 = (bf16_t)(h >> 16);
    l0 = (bf16_t)(l & 0xFFFFu);
    l1 = (bf16_t)(l >> 16);
}

// 16-byte stores through a buffer resource.  A lane whose offset is 2^31 or
// more lies past the resource's range, and the hardware drops its store, so a
// masked store needs no branch: the stores stay straight-line code, and the
// waits for loads issued after them count them exactly.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr uint32_t kDropOffset = 0x80000000u;
template <typename T, int NV>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *v)
{
    constexpr int NW = NV * (int)sizeof(T) / 4;  // dwords
    static_assert(NW % 2 == 0, "whole 8-byte pieces");
    uint32_t w[NW];
#pragma unroll
    for (int e = 0; e < NW; ++e)
        w[e] = sizeof(T) == 4 ? __float_as_uint(v[e]) : pack_bf16x2(v[2 * e], v[2 * e + 1]);
#pragma unroll
    for (int i = 0; i + 4 <= NW; i += 4)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w[i], w[i + 1], w[i + 2], w[i + 3]}, r,
                                               (int)(off + 4 * i), 0, 0);
    if constexpr (NW % 4 == 2)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w[NW - 2], w[NW - 1]}, r,
                                              (int)(off + 4 * (NW - 2)), 0, 0);
}

// NSL: 16-row state slices per workgroup.  With NSL = 4 every operand
// fragment loaded serves four times the matrix work, cutting the operand
// bytes per unit of work (for launches with many sequences, where the bytes
// a CU can keep in flight bound the block rate).  A block takes two phases,
// split by one barrier:
//   1. the row waves form D = U - W S^T and Q Gamma S^T from the same split
//      state fragments, so each is read from LDS once, and publish D^T;
//   2. the row waves add P D to the output and stage it in LDS; the column
//      waves form S Gamma_L + D^T K^ from their fp32 state entries, which
//      stay in registers for the whole call, and write its split over the
//      state the row waves finished reading in phase 1.
// The previous block's outputs leave the staging area as 16-byte stores at
// the start of a block, ahead of its loads: the next block's W, Q Gamma and U
// (into a second register buffer) and this block's P, spread over both
// phases, so the loads are the youngest memory operations when a block
// waits for them.  RAWQ (raw_q_chain): the row waves read the block's q rows
// and the per-token scale s instead of Q Gamma, form Q S^T from two products
// (the q rows exact in bf16, the state split) and scale its rows by s.
template <typename IOT, typename ST, int NSL, bool RAWQ>
__global__ void __launch_bounds__(kChainThreads, 1) prefill_chain_x3_kernel(PrefillArgs a)
{
    constexpr int NR = 16 * NSL;            // state rows of the workgroup
    constexpr int kRowOpsN = 64 + 4 * NSL;  // W 32, Q Gamma 32, U 4 per slice (P apart)
    // 16-byte loads a row wave issues per block: P and half of the next W
    // under phase 1 (kL1, spread over its 24 NSL products), the rest of the
    // next W, Q Gamma and U under phase 2 (kL2, over its 6 NSL products).  The
    // CU's memory queue is then fed through the whole block rather than only
    // while phase 1 runs, and a wave stalls less on a full queue.
    constexpr int kL1 = 8, kL2 = (RAWQ ? 9 : 12) + NSL;
    constexpr int LPS1 = (kL1 + NSL - 1) / NSL, MPL1 = (RAWQ ? 20 : 24) / LPS1;
    constexpr int LPS2 = (kL2 + NSL - 1) / NSL, MPL2 = (6 + LPS2 - 1) / LPS2;
    constexpr int LDO = NR + 4;             // row stride (floats) of the output staging
    constexpr int OPL = NR / 4;             // outputs a lane stores per block
    __shared__ __attribute__((aligned(16))) bf16_t SH[NR][LDKH], SL[NR][LDKH];  // split state
    __shared__ __attribute__((aligned(16))) bf16_t DH[NR][LDJH], DL[NR][LDJH];  // split D^T
    __shared__ __attribute__((aligned(16))) float Ost[4][16][LDO];              // O per row wave

    int n, h, rs;  // rows NR rs .. NR rs + NR - 1
    if (!chain_ids(a, DK / NR, n, h, rs)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int I = wave & 3;
    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    const int start = a.cu[n], end = a.cu[n + 1];
    const int si = a.slot_in[n], so = a.slot_out[n];
    const int row0 = NR * rs;

    if (si >= a.num_rows || so < 0 || so >= a.num_rows) {  // skipped sequence
        for (int idx = tid; idx < (end - start) * NR; idx += kChainThreads) {
            const int t = start + idx / NR, c = row0 + idx % NR;
            st<IOT>(a.out, ((int64_t)t * a.Hv + h) * DK + c, 0.f);
        }
        return;
    }
    const int tb0 = start / CB, tb1 = end > start ? (end - 1) / CB : tb0 - 1;
    const int ntiles = tb1 - tb0 + 1;

    if (wave < 4) {
        if (ntiles <= 0) return;  // nothing to output; the column waves hand the state over
        // W, Q Gamma and U are loaded a block ahead, P (used only after the
        // barrier) at the start of its own block into a single buffer
        auto load_w = [&](int tb, float *ops, int g0) {  // W runs g0 .. g0 + 3
            load_run(ops + 4 * g0, ws.W + ((int64_t)tb * a.Hv + h) * kBlkDK + fidx(8 * I + g0, 0), 4,
                     lane);
        };
        auto load_qu = [&](int tb, float *ops) {
            const int64_t bh = (int64_t)tb * a.Hv + h;
            if constexpr (RAWQ) {
                // ops [32, 48): the q row fragments of steps 0..3 (bf16 bits);
                // [48, 52): s of the lane's four result tokens.  Rows past the
                // input's end repeat its last row (their s is 0).
                const int tok = min(tb * CB + 16 * I + li, a.T - 1);
                const uint4 *qr = reinterpret_cast<const uint4 *>(
                    static_cast<const IOT *>(a.q) + (int64_t)tok * a.q_stride + (h / a.G) * DK + 8 * lq);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint4 w = qr[4 * m];
                    ops[32 + 4 * m] = __uint_as_float(w.x);
                    ops[33 + 4 * m] = __uint_as_float(w.y);
                    ops[34 + 4 * m] = __uint_as_float(w.z);
                    ops[35 + 4 * m] = __uint_as_float(w.w);
                }
                const float4 s4 = *reinterpret_cast<const float4 *>(ws.Qt + bh * kBlkDK + 16 * I + 4 * lq);
                ops[48] = s4.x; ops[49] = s4.y; ops[50] = s4.z; ops[51] = s4.w;
            } else {
                load_run(ops + 32, ws.Qt + bh * kBlkDK + fidx(8 * I, 0), 8, lane);
            }
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl)
                load_run(ops + 64 + 4 * sl, ws.U + bh * kBlkDK + fidx(8 * I + NSL * rs + sl, 0), 1,
                         lane);
        };
        float pb[16];
        // The outputs of block itp, staged by this wave: lane = token lane / 4
        // x a quarter of the workgroup's rows.  Tokens outside the piece, and
        // every lane when itp < 0, take the dropped offset.
        auto flush_o = [&](int itp) {
            const int base = (tb0 + max(itp, 0)) * CB;
            const int p0 = max(start, base) - base, p1 = min(end, base + CB) - base;
            const int tok = lane >> 2, ch = lane & 3, tr = 16 * I + tok;
            float v[OPL];
#pragma unroll
            for (int e = 0; e < OPL; e += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(&Ost[I][tok][ch * OPL + e]);
                v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
            }
            const bool keep = itp >= 0 && tr >= p0 && tr < p1;
            const uint32_t off =
                keep ? (uint32_t)((tr * a.Hv * DK + ch * OPL) * (int)sizeof(IOT)) : kDropOffset;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<IOT *>(a.out) + ((int64_t)base * a.Hv + h) * DK + row0, (short)0,
                p1 * a.Hv * DK * (int)sizeof(IOT), 0x00020000);
            buf_store<IOT, OPL>(r, off, v);
        };
        auto block = [&](int it, const float *cur, float *nxt) {
            const int tb = tb0 + it, base = tb * CB;
            const int p0 = max(start, base) - base, p1 = min(end, base + CB) - base;
            __syncthreads();  // split state in place, last D^T consumed
            flush_o(it - 1);
            load_run(pb, ws.P + ((int64_t)tb * a.Hv + h) * kBlkCB + fidx(4 * I, 0), 4, lane);
            load_w(min(tb + 1, tb1), nxt, 0);
            // phase 1: D = U - W S^T and O = Q Gamma S^T for each slice (ops
            // words [8m, 8m+4) hi, [8m+4, 8m+8) lo of step m); two D
            // accumulators (even / odd steps) halve its dependent chain
            f32x4 oac[NSL];
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {
                const int sr = 16 * sl + li;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc;
                oac[sl] = acc;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const bf16x8_t sh = lds8(&SH[sr][32 * m + 8 * lq]);
                    const bf16x8_t sq = lds8(&SL[sr][32 * m + 8 * lq]);
                    mma3(m & 1 ? acc1 : acc, quad8(cur + 8 * m), quad8(cur + 8 * m + 4), sh, sq);
                    if constexpr (RAWQ) {  // q exact in bf16: no lo part
                        const bf16x8_t qm = quad8(cur + 32 + 4 * m);
                        oac[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm, sq, oac[sl], 0, 0, 0);
                        oac[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qm, sh, oac[sl], 0, 0, 0);
                    } else {
                        mma3(oac[sl], quad8(cur + 32 + 8 * m), quad8(cur + 32 + 8 * m + 4), sh, sq);
                    }
                }
                if constexpr (RAWQ) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) oac[sl][r] *= cur[48 + r];
                }
#pragma unroll
                for (int q = 0; q < LPS1; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MPL1, 0);  // products
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // one load
                }
                acc += acc1;
                float d[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 16 * I + 4 * lq + r;
                    d[r] = (tr >= p0 && tr < p1) ? cur[64 + 4 * sl + r] - acc[r] : 0.f;
                }
                // hi and lo words of the four tokens, two per packed conversion
                const uint32_t h01 = pack_bf16x2(d[0], d[1]), h23 = pack_bf16x2(d[2], d[3]);
                const uint32_t l01 = pack_bf16x2(d[0] - __uint_as_float(h01 << 16),
                                                 d[1] - __uint_as_float(h01 & 0xFFFF0000u));
                const uint32_t l23 = pack_bf16x2(d[2] - __uint_as_float(h23 << 16),
                                                 d[3] - __uint_as_float(h23 & 0xFFFF0000u));
                const int c0 = 16 * I + 4 * lq;
                *reinterpret_cast<uint2 *>(&DH[sr][c0]) = make_uint2(h01, h23);
                *reinterpret_cast<uint2 *>(&DL[sr][c0]) = make_uint2(l01, l23);
            }
            __syncthreads();  // D^T complete
            // phase 2: O += P D, scaled into this wave's staging rows
            load_w(min(tb + 1, tb1), nxt, 4);
            load_qu(min(tb + 1, tb1), nxt);
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {
                const int sr = 16 * sl + li;
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    mma3(oac[sl], quad8(pb + 8 * m), quad8(pb + 8 * m + 4),
                         lds8(&DH[sr][32 * m + 8 * lq]), lds8(&DL[sr][32 * m + 8 * lq]));
#pragma unroll
                for (int q = 0; q < LPS2; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MPL2, 0);  // products
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // one load
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) Ost[I][4 * lq + r][16 * sl + li] = a.scale * oac[sl][r];
            }
        };
        float bufA[kRowOpsN], bufB[kRowOpsN];
        load_w(tb0, bufA, 0);
        load_w(tb0, bufA, 4);
        load_qu(tb0, bufA);
        // pairs of blocks, the odd last block peeled: an exit between the two
        // halves would make the compiler wait for the prefetched operands at
        // the top of every pair
        int it = 0;
        for (; it + 1 < ntiles; it += 2) {
            block(it, bufA, bufB);
            block(it + 1, bufB, bufA);
        }
        if (it < ntiles) block(it, bufA, bufB);
        flush_o(ntiles - 1);
    } else {
        // this lane's fp32 state entries S[16 sl + 4 lq + r][32 I + 16 q + li]
        // (workgroup rows), held in registers from the first block to the last
        // (all loads issued before the first use)
        float sreg[NSL][2][4];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * sl + 4 * lq + r, c = 32 * I + 16 * q + li;
                    sreg[sl][q][r] =
                        ld<ST>(a.ssm_pool, (int64_t)max(si, 0) * a.ssm_stride + ((int64_t)h * DK + row0 + row) * DK + c);
                }
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const int row = 16 * sl + 4 * lq + r, c = 32 * I + 16 * q + li;
                    if (si < 0) sreg[sl][q][r] = sreg[sl][q][r + 1] = 0.f;  // a fresh sequence starts from zero
                    split2(sreg[sl][q][r], sreg[sl][q][r + 1], SH[row][c], SH[row + 1][c], SL[row][c],
                           SL[row + 1][c]);
                }
        auto load_ops = [&](int tb, float *ops) {
            const int pend = min(end, tb * CB + CB) - 1;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = 32 * I + 16 * q + li;
                load_run(ops + 16 * q,
                         ws.KhT + ((int64_t)tb * a.Hv + h) * kBlkDK + fidx(4 * (2 * I + q), 0), 4,
                         lane);
                ops[32 + q] = ws.Ge[((int64_t)pend * a.Hv + h) * DK + c];
            }
        };
        auto block = [&](int it, const float *cur, float *nxt) {
            __syncthreads();
            load_ops(min(tb0 + it + 1, tb1), nxt);  // under phase 1, where these waves wait
            __syncthreads();  // D^T complete; the row waves are done with the state
            // new state columns: S Gamma_L + D^T K^.  The products of both
            // 16-column halves are formed before either is written back, so
            // their matrix-core chains overlap.
            f32x4 acc[2][NSL];
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[q][sl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const bf16x8_t dh = lds8(&DH[16 * sl + li][32 * m + 8 * lq]);
                    const bf16x8_t dl = lds8(&DL[16 * sl + li][32 * m + 8 * lq]);
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        mma3(acc[q][sl], dh, dl, quad8(cur + 16 * q + 8 * m),
                             quad8(cur + 16 * q + 8 * m + 4));
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int c = 32 * I + 16 * q + li;
                const float gm = exp_acc(cur[32 + q]);
#pragma unroll
                for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        const int row = 16 * sl + 4 * lq + r;
                        const float v0 = fmaf(sreg[sl][q][r], gm, acc[q][sl][r]);
                        const float v1 = fmaf(sreg[sl][q][r + 1], gm, acc[q][sl][r + 1]);
                        sreg[sl][q][r] = v0;
                        sreg[sl][q][r + 1] = v1;
                        split2(v0, v1, SH[row][c], SH[row + 1][c], SL[row][c], SL[row + 1][c]);
                    }
            }
        };
        float bufA[kColOps], bufB[kColOps];
        if (ntiles > 0) {
            load_ops(tb0, bufA);
            // pairs of blocks, the odd last block peeled (an exit between the two
            // halves would make the compiler wait for the prefetched operands at
            // the top of every pair)
            int it = 0;
            for (; it + 1 < ntiles; it += 2) {
                block(it, bufA, bufB);
                block(it + 1, bufB, bufA);
            }
            if (it < ntiles) block(it, bufA, bufB);
        }
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * sl + 4 * lq + r, c = 32 * I + 16 * q + li;
                    st<ST>(a.ssm_pool, (int64_t)so * a.ssm_stride + ((int64_t)h * DK + row0 + row) * DK + c,
                           sreg[sl][q][r]);
                }
    }
}

// Compute units of the current device, cached per device: the persistent
// grid of kernel 1 (one workgroup per CU, its LDS allows no more).
static int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <typename IOT, typename ST, bool RAWQ>
static void launch_chain_x3(const PrefillArgs &a, hipStream_t stream)
{
    if ((int64_t)a.N * a.Hv * (DK / 16) <= 384)  // few workgroups: 16 state rows each
        hipLaunchKernelGGL((prefill_chain_x3_kernel<IOT, ST, 1, RAWQ>),
                           dim3(chain_grid(a, DK / 16)), dim3(kChainThreads), 0, stream, a);
    else  // many: 64 state rows per workgroup
        hipLaunchKernelGGL((prefill_chain_x3_kernel<IOT, ST, 4, RAWQ>),
                           dim3(chain_grid(a, DK / 64)), dim3(kChainThreads), 0, stream, a);
}

template <typename IOT, typename ST, int MODE>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    static const bool attr_done = [] {  // opt in to more than 64 KB of LDS per workgroup
        const void *fns[] = {
            reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, true, MODE, false>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, false, MODE, false>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, true, MODE, true>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<IOT, false, MODE, true>)};
        for (const void *f : fns)
            (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kIntraLds);
        return true;
    }();
    (void)attr_done;
    if (a.T > 0) {
        // the persistent grid that loads an item's inputs under the previous one
        const int64_t nitems = (int64_t)((a.T + CB - 1) / CB) * a.Hv;
        const dim3 g1((unsigned)std::min<int64_t>(nitems, cu_count()));
        const dim3 b1(kIntraThreads);
        if (a.kda && a.conv)
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, true, MODE, true>), g1, b1, kIntraLds, stream, a);
        else if (a.kda)
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, true, MODE, false>), g1, b1, kIntraLds, stream, a);
        else if (a.conv)
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, false, MODE, true>), g1, b1, kIntraLds, stream, a);
        else
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, false, MODE, false>), g1, b1, kIntraLds, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (MODE == PM_F32)
        hipLaunchKernelGGL((prefill_chain_kernel<IOT, ST, MODE>), dim3(chain_grid(a, DK / 16)),
                           dim3(kChainThreads), kChainLds, stream, a);
    else if constexpr (std::is_same<IOT, bf16_t>::value) {
        if (!a.kda && !a.conv)  // kernel 1 stored s, not Q Gamma (raw_q_chain)
            launch_chain_x3<IOT, ST, true>(a, stream);
        else
            launch_chain_x3<IOT, ST, false>(a, stream);
    } else {
        launch_chain_x3<IOT, ST, false>(a, stream);
    }
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
