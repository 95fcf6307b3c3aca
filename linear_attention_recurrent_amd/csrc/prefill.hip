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
// with the sequences ("pieces"): kernel 1 works per (tile, head) with a
// same-sequence mask on A and P, so one launch covers every sequence.  The
// cumulative decay G runs continuously over the tile; only differences of G
// between tokens of one piece enter the results.
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
// Every contraction here runs on the matrix cores: v_mfma_f32_16x16x4f32 in
// the fp32 mode.  Lane layout (checked on gfx950): A[i][k] in lane
// i + 16 k, B[k][j] in lane j + 16 k, result D[4 (l/16) + r][l % 16] in
// register r of lane l.
#include "la_device.h"
#include "la_internal.h"

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CB = 64;        // tokens per tile
constexpr int DK = 128;       // head dim (d_k = d_v)
constexpr int LDW = DK + 4;   // LDS row stride (floats) of [64 x 128] arrays
constexpr int LDT = CB + 4;   // LDS row stride of [64 x 64] arrays
constexpr int LDS16 = 16 + 4; // LDS row stride of [64 x 16] arrays
constexpr float kExpClamp = 80.f;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workspace: fp32 arrays indexed by (token, value head).
struct Ws {
    float *U, *W, *Qt, *Kh, *P, *Ge;
};
__host__ __device__ inline Ws ws_layout(void *base, int T, int Hv)
{
    const size_t n = (size_t)T * Hv;
    float *p = static_cast<float *>(base);
    return Ws{p, p + n * DK, p + 2 * n * DK, p + 3 * n * DK, p + 4 * n * DK,
              p + 4 * n * DK + n * CB};
}

size_t prefill_ws_bytes(int N, int T, int Hqk, int Hv, int D, int mode)
{
    (void)N; (void)Hqk; (void)mode;
    if (D != DK || T <= 0) return 0;
    const size_t bytes = (size_t)T * Hv * (5 * DK + CB) * sizeof(float);
    return (bytes + 255) & ~size_t(255);
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

// ---------------------------------------------------------------------------
// Kernel 1: intra-block quantities, one workgroup (4 waves) per (tile, head).
// ---------------------------------------------------------------------------
constexpr size_t kIntraLds =
    (3 * CB * LDW + 2 * CB * LDT + CB + 4 * 16 * 17) * sizeof(float) + 2 * CB * sizeof(int);

template <typename IOT, bool KDA>
__global__ void __launch_bounds__(256) prefill_intra_kernel(PrefillArgs a)
{
    extern __shared__ float sm[];
    float *Xq = sm;                 // q_hat; later beta V, then beta K Gamma
    float *Xk = Xq + CB * LDW;      // k_hat
    float *Gc = Xk + CB * LDW;      // cumulative log decay over the tile
    float *Nm = Gc + CB * LDW;      // N = Diag(beta) A (strictly lower, masked)
    float *Tm = Nm + CB * LDT;      // T = (I + N)^-1
    float *bet = Tm + CB * LDT;     // beta
    float *scr = bet + CB;          // per-wave 16x17 scratch
    int *pst = reinterpret_cast<int *>(scr + 4 * 16 * 17);  // piece start (tile-local)
    int *pen = pst + CB;                                      // piece end (inclusive)

    const int tile = blockIdx.x, h = blockIdx.y, kh = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int t0 = tile * CB;
    const int nt = min(CB, a.T - t0);
    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    auto row = [&](int t) { return ((int64_t)(t0 + t) * a.Hv + h); };

    // 1. token metadata; zero N and T
    if (tid < CB) {
        const int t = tid;
        if (t < nt) {
            const int n = find_seq_p(a.cu, a.N, t0 + t);
            pst[t] = max(a.cu[n], t0) - t0;
            pen[t] = min(a.cu[n + 1], t0 + CB) - 1 - t0;
            bet[t] = a.beta[row(t)];
        } else {
            pst[t] = t;
            pen[t] = t;
            bet[t] = 0.f;
        }
    }
    for (int i = tid; i < CB * LDT; i += 256) {
        Nm[i] = 0.f;
        Tm[i] = 0.f;
    }

    // 2. load and L2-normalise q, k; load g (one wave per token, 2 channels per lane)
    for (int t = wave; t < CB; t += 4) {
        const int c = 2 * lane;
        float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f, g0 = 0.f, g1 = 0.f;
        if (t < nt) {
            const int64_t tok = t0 + t;
            q0 = ld<IOT>(a.q, tok * a.q_stride + kh * DK + c);
            q1 = ld<IOT>(a.q, tok * a.q_stride + kh * DK + c + 1);
            k0 = ld<IOT>(a.k, tok * a.k_stride + kh * DK + c);
            k1 = ld<IOT>(a.k, tok * a.k_stride + kh * DK + c + 1);
            if constexpr (KDA) {
                g0 = a.g[row(t) * DK + c];
                g1 = a.g[row(t) * DK + c + 1];
            } else {
                g0 = g1 = a.g[row(t)];
            }
        }
        const float iq = 1.f / sqrtf(wave_sum(fmaf(q0, q0, q1 * q1)) + a.eps);
        const float ik = 1.f / sqrtf(wave_sum(fmaf(k0, k0, k1 * k1)) + a.eps);
        Xq[t * LDW + c] = q0 * iq;
        Xq[t * LDW + c + 1] = q1 * iq;
        Xk[t * LDW + c] = k0 * ik;
        Xk[t * LDW + c + 1] = k1 * ik;
        Gc[t * LDW + c] = g0;
        Gc[t * LDW + c + 1] = g1;
    }
    __syncthreads();
    if (tid < DK) {  // cumulative sum over the tile, per channel
        float run = 0.f;
        for (int t = 0; t < CB; ++t) {
            run += Gc[t * LDW + tid];
            Gc[t * LDW + tid] = run;
        }
    }
    __syncthreads();

    // 3. Q Gamma, K Gamma_L / Gamma and the piece's total log decay
    for (int idx = tid; idx < nt * DK; idx += 256) {
        const int t = idx / DK, c = idx % DK;
        const float G = Gc[t * LDW + c];
        const float Gs = pst[t] > 0 ? Gc[(pst[t] - 1) * LDW + c] : 0.f;
        const float Ge = Gc[pen[t] * LDW + c];
        const int64_t o = row(t) * DK + c;
        ws.Qt[o] = Xq[t * LDW + c] * expf(G - Gs);
        ws.Kh[o] = Xk[t * LDW + c] * expf(Ge - G);
        if (t == pen[t]) ws.Ge[o] = Ge - Gs;
    }

    // 4. A and P, tile by tile on the matrix cores.  Wave jobs: row sub-block
    //    I with column sub-blocks [Jlo, Jhi].
    {
        int I, Jlo, Jhi;
        if (wave == 0) { I = 3; Jlo = 0; Jhi = 1; }
        else if (wave == 1) { I = 3; Jlo = 2; Jhi = 3; }
        else if (wave == 2) { I = 2; Jlo = 0; Jhi = 2; }
        else { I = 1; Jlo = 0; Jhi = 1; }
        for (int pass = 0; pass < (wave == 3 ? 2 : 1); ++pass) {
            if (pass == 1) { I = 0; Jlo = 0; Jhi = 0; }
            f32x4 accA[3], accP[3];
            for (int q = 0; q < 3; ++q) {
                accA[q] = f32x4{0.f, 0.f, 0.f, 0.f};
                accP[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const int t = 16 * I + li;
            for (int k0 = 0; k0 < DK; k0 += 4) {
                const int c = k0 + lk;
                const float R = I ? Gc[(16 * I - 1) * LDW + c] : 0.f;
                const float et = expf(fminf(Gc[t * LDW + c] - R, kExpClamp));
                const float at = Xk[t * LDW + c] * et, aq = Xq[t * LDW + c] * et;
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const int J = Jlo + q;
                    if (J <= Jhi) {
                        const int j = 16 * J + li;
                        const float bj = Xk[j * LDW + c] * expf(fminf(R - Gc[j * LDW + c], kExpClamp));
                        accA[q] = mfma4(at, bj, accA[q]);
                        accP[q] = mfma4(aq, bj, accP[q]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int J = Jlo + q;
                if (J > Jhi) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = 16 * I + 4 * lk + r, j = 16 * J + li;
                    const bool same = j >= pst[tt] && tt < nt;
                    Nm[tt * LDT + j] = (same && j < tt) ? bet[tt] * accA[q][r] : 0.f;
                    if (tt < nt) ws.P[row(tt) * CB + j] = (same && j <= tt) ? accP[q][r] : 0.f;
                }
            }
        }
        // the upper tiles of P are zero
        for (int idx = tid; idx < nt * CB; idx += 256) {
            const int tt = idx / CB, j = idx % CB;
            if ((j >> 4) > (tt >> 4)) ws.P[row(tt) * CB + j] = 0.f;
        }
    }
    __syncthreads();

    // 5. T = (I + N)^-1.  Diagonal 16x16 blocks by forward substitution (one
    //    wave per block, lane c < 16 holds column c), then the off-diagonal
    //    blocks level by level: T_IJ = -T_II sum_{K=J}^{I-1} N_IK T_KJ.
    {
        const int I = wave;
        if (lane < 16) {
            const int c = lane;
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < t; ++j) s = fmaf(Nm[(16 * I + t) * LDT + 16 * I + j], x[j], s);
                x[t] = t == c ? 1.f : (t < c ? 0.f : -s);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Tm[(16 * I + t) * LDT + 16 * I + c] = x[t];
        }
    }
    __syncthreads();
    float *ws16 = scr + wave * 16 * 17;
    for (int lev = 1; lev <= 3; ++lev) {
        const int I = wave, J = wave - lev;
        if (J >= 0) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K)
                for (int k0 = 0; k0 < 16; k0 += 4)
                    acc = mfma4(Nm[(16 * I + li) * LDT + 16 * K + k0 + lk],
                                Tm[(16 * K + k0 + lk) * LDT + 16 * J + li], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) ws16[(4 * lk + r) * 17 + li] = acc[r];
            __builtin_amdgcn_wave_barrier();
            f32x4 t2 = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < 16; k0 += 4)
                t2 = mfma4(Tm[(16 * I + li) * LDT + 16 * I + k0 + lk], ws16[(k0 + lk) * 17 + li], t2);
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(16 * I + 4 * lk + r) * LDT + 16 * J + li] = -t2[r];
        }
        __syncthreads();
    }

    // 6. U = T (beta V) and 7. W = T (beta K Gamma), 16-column tiles, two per wave
    for (int which = 0; which < 2; ++which) {
        for (int idx = tid; idx < CB * DK; idx += 256) {
            const int t = idx / DK, c = idx % DK;
            float x = 0.f;
            if (t < nt) {
                if (which == 0) {
                    x = ld<IOT>(a.v, (int64_t)(t0 + t) * a.v_stride + h * DK + c);
                } else {
                    const float Gs = pst[t] > 0 ? Gc[(pst[t] - 1) * LDW + c] : 0.f;
                    x = Xk[t * LDW + c] * expf(Gc[t * LDW + c] - Gs);
                }
                x *= bet[t];
            }
            Xq[t * LDW + c] = x;
        }
        __syncthreads();
        float *dst = which ? ws.W : ws.U;
        for (int C = 2 * wave; C < 2 * wave + 2; ++C) {
            for (int I = 0; I < 4; ++I) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < 16 * (I + 1); k0 += 4)
                    acc = mfma4(Tm[(16 * I + li) * LDT + k0 + lk], Xq[(k0 + lk) * LDW + 16 * C + li],
                                acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * I + 4 * lk + r;
                    if (t < nt) dst[row(t) * DK + 16 * C + li] = acc[r];
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: the block chain, one workgroup per (sequence, head, 16 state rows).
// ---------------------------------------------------------------------------
constexpr size_t kChainLds =
    (3 * CB * LDW + CB * LDT + 2 * CB * LDS16 + 16 * LDW + DK) * sizeof(float);

template <typename IOT, typename ST>
__global__ void __launch_bounds__(256) prefill_chain_kernel(PrefillArgs a)
{
    extern __shared__ float sm[];
    float *Wl = sm;                  // W rows of the block
    float *Ql = Wl + CB * LDW;       // Q Gamma
    float *Kl = Ql + CB * LDW;       // K Gamma_L / Gamma
    float *Pl = Kl + CB * LDW;       // P (block-local columns)
    float *Ul = Pl + CB * LDT;       // U, this slice's 16 columns
    float *Dl = Ul + CB * LDS16;     // D, this slice's 16 columns
    float *St = Dl + CB * LDS16;     // state slice [16 rows x 128]
    float *gam = St + 16 * LDW;      // Gamma_L of the block

    const int n = blockIdx.x, h = blockIdx.y, rs = blockIdx.z;  // rows 16 rs .. 16 rs + 15
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const Ws ws = ws_layout(a.ws, a.T, a.Hv);
    const int start = a.cu[n], end = a.cu[n + 1];
    const int si = a.slot_in[n], so = a.slot_out[n];

    if (si >= a.num_rows || so < 0 || so >= a.num_rows) {  // skipped sequence
        for (int idx = tid; idx < (end - start) * 16; idx += 256) {
            const int t = start + idx / 16, c = 16 * rs + idx % 16;
            st<IOT>(a.out, ((int64_t)t * a.Hv + h) * DK + c, 0.f);
        }
        return;
    }
    // initial state slice
    for (int idx = tid; idx < 16 * DK; idx += 256) {
        const int i = idx / DK, c = idx % DK;
        float v = 0.f;
        if (si >= 0)
            v = ld<ST>(a.ssm_pool,
                       (int64_t)si * a.ssm_stride + ((int64_t)h * DK + 16 * rs + i) * DK + c);
        St[i * LDW + c] = v;
    }

    for (int tile = start / CB; start < end && tile <= (end - 1) / CB; ++tile) {
        const int pa = max(start, tile * CB), pb = min(end, tile * CB + CB);
        const int L = pb - pa, p0 = pa - tile * CB;
        __syncthreads();  // previous block done with the LDS operands
        // a. stage the block's operands (rows >= L zero)
        for (int idx = tid; idx < CB * (DK / 4); idx += 256) {
            const int t = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
            float4 w4 = {0.f, 0.f, 0.f, 0.f}, q4 = w4, k4 = w4;
            if (t < L) {
                const int64_t o = ((int64_t)(pa + t) * a.Hv + h) * DK + c4;
                w4 = *reinterpret_cast<const float4 *>(ws.W + o);
                q4 = *reinterpret_cast<const float4 *>(ws.Qt + o);
                k4 = *reinterpret_cast<const float4 *>(ws.Kh + o);
            }
            *reinterpret_cast<float4 *>(Wl + t * LDW + c4) = w4;
            *reinterpret_cast<float4 *>(Ql + t * LDW + c4) = q4;
            *reinterpret_cast<float4 *>(Kl + t * LDW + c4) = k4;
        }
        for (int idx = tid; idx < CB * CB; idx += 256) {
            const int t = idx / CB, j = idx % CB;
            Pl[t * LDT + j] = (t < L && j < L) ? ws.P[((int64_t)(pa + t) * a.Hv + h) * CB + p0 + j]
                                               : 0.f;
        }
        for (int idx = tid; idx < CB * 16; idx += 256) {
            const int t = idx / 16, c = idx % 16;
            Ul[t * LDS16 + c] =
                t < L ? ws.U[((int64_t)(pa + t) * a.Hv + h) * DK + 16 * rs + c] : 0.f;
        }
        if (tid < DK) gam[tid] = expf(ws.Ge[((int64_t)(pb - 1) * a.Hv + h) * DK + tid]);
        __syncthreads();

        // b. D = U - W S^T  (wave I: token rows 16I .. 16I + 15)
        const int I = wave;
        if (16 * I < L) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < DK; k0 += 4)
                acc = mfma4(Wl[(16 * I + li) * LDW + k0 + lk], St[li * LDW + k0 + lk], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lk + r;
                Dl[t * LDS16 + li] = Ul[t * LDS16 + li] - acc[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) Dl[(16 * I + 4 * lk + r) * LDS16 + li] = 0.f;
        }
        __syncthreads();

        // c. O = scale (Q S^T + P D) for rows 16I.., and the new state columns
        if (16 * I < L) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < DK; k0 += 4)
                acc = mfma4(Ql[(16 * I + li) * LDW + k0 + lk], St[li * LDW + k0 + lk], acc);
            for (int k0 = 0; k0 < 16 * (I + 1); k0 += 4)
                acc = mfma4(Pl[(16 * I + li) * LDT + k0 + lk], Dl[(k0 + lk) * LDS16 + li], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * I + 4 * lk + r;
                if (t < L)
                    st<IOT>(a.out, ((int64_t)(pa + t) * a.Hv + h) * DK + 16 * rs + li,
                            a.scale * acc[r]);
            }
        }
        f32x4 snew[2];
        for (int q = 0; q < 2; ++q) {
            const int C = 2 * wave + q;  // state columns 16C .. 16C + 15
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < L; k0 += 4)
                acc = mfma4(Dl[(k0 + lk) * LDS16 + li], Kl[(k0 + lk) * LDW + 16 * C + li], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * lk + r, c = 16 * C + li;
                acc[r] = fmaf(St[i * LDW + c], gam[c], acc[r]);
            }
            snew[q] = acc;
        }
        __syncthreads();  // every wave is done reading the old state
        for (int q = 0; q < 2; ++q) {
            const int C = 2 * wave + q;
#pragma unroll
            for (int r = 0; r < 4; ++r) St[(4 * lk + r) * LDW + 16 * C + li] = snew[q][r];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * DK; idx += 256) {
        const int i = idx / DK, c = idx % DK;
        st<ST>(a.ssm_pool, (int64_t)so * a.ssm_stride + ((int64_t)h * DK + 16 * rs + i) * DK + c,
               St[i * LDW + c]);
    }
}

template <typename IOT, typename ST>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    if (a.T > 0) {
        const dim3 g1((unsigned)((a.T + CB - 1) / CB), (unsigned)a.Hv);
        if (a.kda)
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, true>), g1, dim3(256), kIntraLds, stream, a);
        else
            hipLaunchKernelGGL((prefill_intra_kernel<IOT, false>), g1, dim3(256), kIntraLds, stream,
                               a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 g2((unsigned)a.N, (unsigned)a.Hv, (unsigned)(DK / 16));
    hipLaunchKernelGGL((prefill_chain_kernel<IOT, ST>), g2, dim3(256), kChainLds, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.mode != 0) return hipErrorNotSupported;  // bf16-operand mode not built yet
    static const bool attr_done = [] {  // opt in to more than 64 KB of LDS per workgroup
        const void *ks[] = {
            reinterpret_cast<const void *>(&prefill_intra_kernel<float, true>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<float, false>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<bf16_t, true>),
            reinterpret_cast<const void *>(&prefill_intra_kernel<bf16_t, false>)};
        for (const void *k : ks)
            (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)kIntraLds);
        const void *kc[] = {
            reinterpret_cast<const void *>(&prefill_chain_kernel<float, float>),
            reinterpret_cast<const void *>(&prefill_chain_kernel<float, bf16_t>),
            reinterpret_cast<const void *>(&prefill_chain_kernel<bf16_t, float>),
            reinterpret_cast<const void *>(&prefill_chain_kernel<bf16_t, bf16_t>)};
        for (const void *k : kc)
            (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)kChainLds);
        return true;
    }();
    (void)attr_done;
    const int code = (a.io_dtype ? 2 : 0) | (a.state_dtype ? 1 : 0);
    switch (code) {
    case 0: return launch_prefill_t<float, float>(a, stream);
    case 1: return launch_prefill_t<float, bf16_t>(a, stream);
    case 2: return launch_prefill_t<bf16_t, float>(a, stream);
    default: return launch_prefill_t<bf16_t, bf16_t>(a, stream);
    }
}

}  // namespace la
