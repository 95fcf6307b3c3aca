/*
 * oracle.c -- plain, sequential, fp64 CPU oracle for the linear-attention
 * recurrent-state path (Kimi Delta Attention and Gated DeltaNet decode and
 * prefill, with the kernel-size-4 depthwise causal short conv).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, helper or constant
 * with the HIP library; its inputs arrive as fp64 arrays (exact copies of the
 * stored bf16/fp32 values) and it rounds to the storage dtype with its own
 * codec below.
 *
 * Every function is the plain definition written out, token by token, with no
 * blocking, fusion or reordering.  Sources (the pages):
 *   [SGLang-pool]  "SGLang之KV Cache内存池机制" (yuyanqi.com), section 8.2
 *                  (state shapes and pool layout) and section 8.5 (the decode
 *                  kernel's steps: load state, decay by exp(g), delta
 *                  correction, beta gating, rank-1 update, output, write-back;
 *                  extend reads the initial state from the pool and writes the
 *                  final state back in place).
 *   [mamba-ish]    xxmr.cn/news/181459, the "Conv state" passage (depthwise
 *                  causal short conv, kernel 4, keep the last 3 inputs), the
 *                  "KDA recurrent update" passage (alpha is per key channel
 *                  for KDA, a scalar per head for GDN) and the ReplaySSM
 *                  exact-commit passage (k = rawk / sqrt(|rawk|^2 + eps),
 *                  alpha = exp(g), S <- S Diag(alpha), d = beta (v - S k),
 *                  S <- S + d k^T); the ReplaySSM verify/commit passages
 *                  (per-step outputs from the checkpoint, a per-slot ring of
 *                  step records, replay of the accepted prefix) and the
 *                  "intermediate_conv_window" passage (per-step conv history).
 *   [deploy]       hotelren.com/news/5417338 section 2.1 (state [H, d_v, d_k]
 *                  accumulating v k^T; conv state keeps the last 3 q/k/v
 *                  projections).
 * Readings where the pages are silent (all passed in or fixed here):
 *   - state orientation [H, d_v, d_k], d_k contiguous;
 *   - channel order of x / conv state: [Q heads | K heads | V heads],
 *     head-major inside each block;
 *   - conv is a cross-correlation: tap 3 multiplies the current token,
 *     conv-state row 0 is the oldest token;
 *   - SiLU after the conv on every channel; optional bias;
 *   - q is L2-normalised like k, with the same eps form;
 *   - the output uses the post-update state, times `scale`;
 *   - GQA: value head h reads q/k head floor(h / (H_v / H_qk)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Storage dtypes the oracle rounds to. */
enum { ORC_FP32 = 0, ORC_BF16 = 1, ORC_FP64 = 2 };

/* ------------------------------------------------------------------ */
/* Rounding codec (independent of any GPU conversion).                */
/* ------------------------------------------------------------------ */

/* Round an fp64 value to the nearest bf16 value, ties to even.
 * bf16 = 1 sign bit, 8 exponent bits (same range as fp32), 8 significant
 * bits.  Works in the value domain: the quantum of a bf16 number with
 * binade exponent e (|x| in [2^(e-1), 2^e)) is 2^(e-8); below the normal
 * range the quantum stays at the subnormal spacing 2^-133. */
static double round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                       /* |x| = m * 2^e, m in [0.5, 1) */
    if (e < -125) e = -125;             /* subnormal bf16 spacing */
    double quantum = ldexp(1.0, e - 8);
    double r = nearbyint(x / quantum) * quantum; /* current mode: ties-to-even */
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) return copysign(INFINITY, x);
    return r;
}

double orc_round(double x, int dtype)
{
    switch (dtype) {
    case ORC_FP32: return (double)(float)x; /* C conversion rounds to nearest-even */
    case ORC_BF16: return round_bf16(x);
    default: return x;
    }
}

void orc_round_array(double *x, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) x[i] = orc_round(x[i], dtype);
}

static double silu(double y) { return y / (1.0 + exp(-y)); }

/* ------------------------------------------------------------------ */
/* Short conv, one decode token ([mamba-ish] "Conv state" passage;    */
/* [SGLang-pool] 8.5 step 1, in-place update of the indexed rows).    */
/* ------------------------------------------------------------------ */

/* One token per batch entry.  x [B, C]; w [C, 4]; bias [C] or NULL;
 * conv_pool rows [3, C] at conv_pool + slot * conv_stride.
 * y [B, C] receives SiLU(sum_i w[c,i] * window[i] + bias[c]) in fp64 (not
 * rounded; callers round to their output dtype).  The conv state is rolled:
 * rows 1, 2 move to 0, 1 and the current input becomes row 2, rounded to
 * conv_dtype (a plain copy when x already has that dtype). */
void orc_shortconv_step(int B, int C, const double *x, const double *w,
                        const double *bias, double *conv_pool,
                        int64_t conv_stride, int conv_dtype,
                        const int32_t *slots, double *y)
{
    for (int b = 0; b < B; ++b) {
        double *cs = conv_pool + (int64_t)slots[b] * conv_stride;
        for (int c = 0; c < C; ++c) {
            double win[4] = {cs[c], cs[C + c], cs[2 * C + c], x[(int64_t)b * C + c]};
            double acc = bias ? bias[c] : 0.0;
            for (int i = 0; i < 4; ++i) acc += w[4 * c + i] * win[i];
            y[(int64_t)b * C + c] = silu(acc);
            cs[c] = win[1];
            cs[C + c] = win[2];
            cs[2 * C + c] = orc_round(win[3], conv_dtype);
        }
    }
}

/* ------------------------------------------------------------------ */
/* The gated delta rule, one token for one (entry, value head).       */
/* ------------------------------------------------------------------ */

/* L2 normalisation x / sqrt(sum x^2 + eps) ([mamba-ish] ReplaySSM
 * exact-commit passage, applied to k and, by the same form, to q). */
static void l2norm(const double *in, double *out, int n, double eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += in[i] * in[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) out[i] = in[i] * inv;
}

/* S [dv, dk] (row i = value channel i) is updated in place:
 *   S <- S Diag(alpha);  d = beta (v - S k);  S <- S + d k^T;  o = scale S q.
 * q, k are already normalised; alpha has dk entries. */
static void delta_rule_token_d(double *S, int dk, int dv, const double *q,
                               const double *k, const double *v,
                               const double *alpha, double beta, double scale,
                               double *o, double *dvec)
{
    for (int i = 0; i < dv; ++i) {
        double *row = S + (int64_t)i * dk;
        for (int c = 0; c < dk; ++c) row[c] *= alpha[c];
        double u = 0.0;
        for (int c = 0; c < dk; ++c) u += row[c] * k[c];
        double d = beta * (v[i] - u);
        for (int c = 0; c < dk; ++c) row[c] += d * k[c];
        if (dvec) dvec[i] = d;
        if (!o) continue;
        double p = 0.0;
        for (int c = 0; c < dk; ++c) p += row[c] * q[c];
        o[i] = scale * p;
    }
}

static void delta_rule_token(double *S, int dk, int dv, const double *q,
                             const double *k, const double *v,
                             const double *alpha, double beta, double scale,
                             double *o)
{
    delta_rule_token_d(S, dk, dv, q, k, v, alpha, beta, scale, o, NULL);
}

/* Decode recurrence for one token per entry.
 * q, k [B, Hqk, dk] and v [B, Hv, dv] are the raw (pre-normalisation) vectors.
 * KDA (kda=1): g [B, Hv, dk] log-decays, one per key channel.
 * GDN (kda=0): g [B, Hv], one scalar per value head.
 * beta [B, Hv].  ssm_pool rows [Hv, dv, dk] at ssm_pool + slot * ssm_stride;
 * each row is read, advanced in fp64, and stored rounded to state_dtype.
 * out [B, Hv, dv] is rounded to io_dtype. */
int orc_recurrent_step(int kda, int B, int Hqk, int Hv, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const int32_t *slots, double *ssm_pool,
                       int64_t ssm_stride, int state_dtype, double *out,
                       int io_dtype, double eps, double scale)
{
    if (Hqk <= 0 || Hv % Hqk != 0) return -1;
    const int group = Hv / Hqk;
    double *qn = malloc(sizeof(double) * dk), *kn = malloc(sizeof(double) * dk);
    double *alpha = malloc(sizeof(double) * dk), *o = malloc(sizeof(double) * dv);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hv; ++h) {
            const int kh = h / group;
            l2norm(q + ((int64_t)b * Hqk + kh) * dk, qn, dk, eps);
            l2norm(k + ((int64_t)b * Hqk + kh) * dk, kn, dk, eps);
            for (int c = 0; c < dk; ++c)
                alpha[c] = exp(kda ? g[((int64_t)b * Hv + h) * dk + c] : g[(int64_t)b * Hv + h]);
            double *S = ssm_pool + (int64_t)slots[b] * ssm_stride + (int64_t)h * dv * dk;
            delta_rule_token(S, dk, dv, qn, kn, v + ((int64_t)b * Hv + h) * dv, alpha,
                             beta[(int64_t)b * Hv + h], scale, o);
            for (int i = 0; i < dv * dk; ++i) S[i] = orc_round(S[i], state_dtype);
            for (int i = 0; i < dv; ++i)
                out[((int64_t)b * Hv + h) * dv + i] = orc_round(o[i], io_dtype);
        }
    }
    free(qn); free(kn); free(alpha); free(o);
    return 0;
}

/* Full decode step: the short conv + SiLU over x [B, C] (skipped when
 * w == NULL, then x already holds the post-conv q|k|v), the split into
 * q [Hqk, dk] | k [Hqk, dk] | v [Hv, dv], then the recurrence.  The post-conv
 * q/k/v stay in fp64 (never rounded to the I/O dtype). */
int orc_decode(int kda, int B, int Hqk, int Hv, int dk, int dv,
               const double *x, const double *w, const double *bias,
               double *conv_pool, int64_t conv_stride, int conv_dtype,
               const double *g, const double *beta, const int32_t *slots,
               double *ssm_pool, int64_t ssm_stride, int state_dtype,
               double *out, int io_dtype, double eps, double scale)
{
    const int C = 2 * Hqk * dk + Hv * dv;
    double *y = malloc(sizeof(double) * (size_t)B * C);
    if (w) orc_shortconv_step(B, C, x, w, bias, conv_pool, conv_stride, conv_dtype, slots, y);
    else memcpy(y, x, sizeof(double) * (size_t)B * C);
    double *q = malloc(sizeof(double) * (size_t)B * Hqk * dk);
    double *k = malloc(sizeof(double) * (size_t)B * Hqk * dk);
    double *v = malloc(sizeof(double) * (size_t)B * Hv * dv);
    for (int b = 0; b < B; ++b) {
        const double *yb = y + (int64_t)b * C;
        memcpy(q + (int64_t)b * Hqk * dk, yb, sizeof(double) * Hqk * dk);
        memcpy(k + (int64_t)b * Hqk * dk, yb + Hqk * dk, sizeof(double) * Hqk * dk);
        memcpy(v + (int64_t)b * Hv * dv, yb + 2 * Hqk * dk, sizeof(double) * Hv * dv);
    }
    int rc = orc_recurrent_step(kda, B, Hqk, Hv, dk, dv, q, k, v, g, beta, slots, ssm_pool,
                                ssm_stride, state_dtype, out, io_dtype, eps, scale);
    free(y); free(q); free(k); free(v);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Prefill over packed variable-length sequences ([SGLang-pool] 8.5,  */
/* extend: initial state read from the pool, final state written     */
/* back; the method's result is the same recurrence token by token).  */
/* ------------------------------------------------------------------ */

/* Short conv over packed sequences.  Sequence n covers tokens
 * [cu[n], cu[n+1]) of x [T, C].  Its history comes from conv_pool row
 * slot_in[n] (zeros when slot_in[n] < 0); after the last token the three most
 * recent pre-conv inputs (older history shifted in for sequences shorter than
 * three tokens) are stored to row slot_out[n], rounded to conv_dtype.  Inside
 * the call the window holds the sequence's own inputs; the stored history only
 * supplies the positions before the sequence's first token.  y [T, C] gets the
 * SiLU output rounded to io_dtype. */
void orc_shortconv_prefill(int N, int C, const double *x, const int32_t *cu,
                           const int32_t *slot_in, const int32_t *slot_out,
                           const double *w, const double *bias,
                           double *conv_pool, int64_t conv_stride,
                           int conv_dtype, double *y, int io_dtype)
{
    double *hist = malloc(sizeof(double) * 3 * (size_t)C);
    for (int n = 0; n < N; ++n) {
        if (slot_in[n] >= 0)
            memcpy(hist, conv_pool + (int64_t)slot_in[n] * conv_stride, sizeof(double) * 3 * C);
        else
            memset(hist, 0, sizeof(double) * 3 * (size_t)C);
        for (int t = cu[n]; t < cu[n + 1]; ++t) {
            for (int c = 0; c < C; ++c) {
                double win[4] = {hist[c], hist[C + c], hist[2 * C + c], x[(int64_t)t * C + c]};
                double acc = bias ? bias[c] : 0.0;
                for (int i = 0; i < 4; ++i) acc += w[4 * c + i] * win[i];
                y[(int64_t)t * C + c] = orc_round(silu(acc), io_dtype);
                hist[c] = win[1];
                hist[C + c] = win[2];
                hist[2 * C + c] = win[3];  /* inside the call the window holds the inputs */
            }
        }
        /* only the hand-off to the next call is stored in the conv dtype */
        for (int64_t i = 0; i < 3 * (int64_t)C; ++i)
            conv_pool[(int64_t)slot_out[n] * conv_stride + i] = orc_round(hist[i], conv_dtype);
    }
    free(hist);
}

/* Recurrent-state prefill over packed sequences.  q, k [T, Hqk, dk] and
 * v [T, Hv, dv] with token strides q_stride, k_stride, v_stride (elements);
 * g [T, Hv, dk] (KDA) or [T, Hv] (GDN); beta [T, Hv]; out [T, Hv, dv].
 * The state starts from pool row slot_in[n] (zero when slot_in[n] < 0), is
 * carried in fp64 over the whole sequence, and is rounded to state_dtype only
 * when written to row slot_out[n]. */
int orc_prefill(int kda, int N, int Hqk, int Hv, int dk, int dv,
                const double *q, int64_t q_stride, const double *k,
                int64_t k_stride, const double *v, int64_t v_stride,
                const double *g, const double *beta, const int32_t *cu,
                const int32_t *slot_in, const int32_t *slot_out,
                double *ssm_pool, int64_t ssm_stride, int state_dtype,
                double *out, int io_dtype, double eps, double scale)
{
    if (Hqk <= 0 || Hv % Hqk != 0) return -1;
    const int group = Hv / Hqk;
    const size_t state_elems = (size_t)Hv * dv * dk;
    double *S = malloc(sizeof(double) * state_elems);
    double *qn = malloc(sizeof(double) * dk), *kn = malloc(sizeof(double) * dk);
    double *alpha = malloc(sizeof(double) * dk), *o = malloc(sizeof(double) * dv);
    for (int n = 0; n < N; ++n) {
        if (slot_in[n] >= 0)
            memcpy(S, ssm_pool + (int64_t)slot_in[n] * ssm_stride, sizeof(double) * state_elems);
        else
            memset(S, 0, sizeof(double) * state_elems);
        for (int t = cu[n]; t < cu[n + 1]; ++t) {
            for (int h = 0; h < Hv; ++h) {
                const int kh = h / group;
                l2norm(q + (int64_t)t * q_stride + (int64_t)kh * dk, qn, dk, eps);
                l2norm(k + (int64_t)t * k_stride + (int64_t)kh * dk, kn, dk, eps);
                for (int c = 0; c < dk; ++c)
                    alpha[c] = exp(kda ? g[((int64_t)t * Hv + h) * dk + c] : g[(int64_t)t * Hv + h]);
                delta_rule_token(S + (size_t)h * dv * dk, dk, dv, qn, kn,
                                 v + (int64_t)t * v_stride + (int64_t)h * dv, alpha,
                                 beta[(int64_t)t * Hv + h], scale, o);
                for (int i = 0; i < dv; ++i)
                    out[((int64_t)t * Hv + h) * dv + i] = orc_round(o[i], io_dtype);
            }
        }
        double *dst = ssm_pool + (int64_t)slot_out[n] * ssm_stride;
        for (size_t i = 0; i < state_elems; ++i) dst[i] = orc_round(S[i], state_dtype);
    }
    free(S); free(qn); free(kn); free(alpha); free(o);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Speculative verify and exact commit ([mamba-ish] ReplaySSM         */
/* passages: verify computes every draft step's output from the       */
/* checkpoint without writing the state back and appends the step's   */
/* record to a per-slot ring of depth L; the commit replays the       */
/* accepted prefix from the checkpoint with k = rawk/sqrt(|rawk|^2 +  */
/* eps), alpha = exp(g), S <- S Diag(alpha), d = beta (rawv - S k),   */
/* S <- S + d k^T, and writes the result back).                       */
/* ------------------------------------------------------------------ */

/* Ring layout, per pool row (slot): [num_rows, Hv, L, n] for the vectors
 * (d and rawv: n = dv; k and rawk: n = dk; g: n = dk for KDA, 1 for GDN) and
 * [num_rows, Hv, L] for beta.  Draft step t of request b lives at position
 * (ring_base[b] + t) mod L.  d, k, rawv, rawk are stored rounded to io_dtype;
 * g and beta keep their fp32 input values. */
static int64_t ring_at(int slot, int Hv, int L, int h, int pos, int n)
{
    return (((int64_t)slot * Hv + h) * L + pos) * n;
}

/* x [B, D, C] pre-conv inputs of up to D draft tokens per request (n_tok[b]
 * of them used); g [B, D, Hv, dk] (KDA) or [B, D, Hv]; beta [B, D, Hv].
 * For each request, from the conv history and state of pool row slots[b]
 * (neither is modified): token by token, the short conv + SiLU (the output
 * rounded to io_dtype, as a separate conv kernel would store it), the split
 * into q | k | v, the L2 norms, and the gated delta rule with the state
 * carried in fp64 across the tokens.  out [B, D, Hv, dv] gets each step's
 * output (zeros past n_tok[b]); windows [B, D, 3, C] the conv history after
 * each step (what the conv pool would hold had that step been the last
 * accepted one).  w == NULL: x already holds the post-conv q|k|v and windows
 * is not written. */
int orc_verify(int kda, int B, int D, const int32_t *n_tok, int Hqk, int Hv, int dk, int dv,
               const double *x, const double *w, const double *bias,
               const double *conv_pool, int64_t conv_stride, int conv_dtype,
               const double *g, const double *beta, const int32_t *slots,
               const double *ssm_pool, int64_t ssm_stride,
               double *out, int io_dtype, double *windows,
               int L, const int32_t *ring_base, double *ring_d, double *ring_k,
               double *ring_g, double *ring_rawv, double *ring_rawk, double *ring_beta,
               double eps, double scale)
{
    if (Hqk <= 0 || Hv % Hqk != 0) return -1;
    const int group = Hv / Hqk;
    const int C = 2 * Hqk * dk + Hv * dv;
    const size_t state_elems = (size_t)Hv * dv * dk;
    double *S = malloc(sizeof(double) * state_elems);
    double *hist = malloc(sizeof(double) * 3 * (size_t)C);
    double *y = malloc(sizeof(double) * (size_t)C);
    double *qn = malloc(sizeof(double) * dk), *kn = malloc(sizeof(double) * dk);
    double *alpha = malloc(sizeof(double) * dk), *o = malloc(sizeof(double) * dv);
    double *dd = malloc(sizeof(double) * dv);
    for (int b = 0; b < B; ++b) {
        const int slot = slots[b];
        memcpy(S, ssm_pool + (int64_t)slot * ssm_stride, sizeof(double) * state_elems);
        if (w) memcpy(hist, conv_pool + (int64_t)slot * conv_stride, sizeof(double) * 3 * C);
        for (int t = 0; t < D; ++t) {
            double *ob = out + ((int64_t)b * D + t) * Hv * dv;
            if (t >= n_tok[b]) {
                memset(ob, 0, sizeof(double) * (size_t)Hv * dv);
                continue;
            }
            const double *xt = x + ((int64_t)b * D + t) * C;
            if (w) {
                for (int c = 0; c < C; ++c) {
                    double win[4] = {hist[c], hist[C + c], hist[2 * C + c], xt[c]};
                    double acc = bias ? bias[c] : 0.0;
                    for (int i = 0; i < 4; ++i) acc += w[4 * c + i] * win[i];
                    y[c] = orc_round(silu(acc), io_dtype);
                    hist[c] = win[1];
                    hist[C + c] = win[2];
                    hist[2 * C + c] = orc_round(win[3], conv_dtype);
                }
                memcpy(windows + ((int64_t)b * D + t) * 3 * C, hist, sizeof(double) * 3 * C);
            } else {
                memcpy(y, xt, sizeof(double) * C);
            }
            const int pos = (ring_base[b] + t) & (L - 1);
            for (int h = 0; h < Hv; ++h) {
                const int kh = h / group;
                const double *qr = y + kh * dk, *kr = y + Hqk * dk + kh * dk;
                const double *vr = y + 2 * Hqk * dk + h * dv;
                l2norm(qr, qn, dk, eps);
                l2norm(kr, kn, dk, eps);
                const double *gt = kda ? g + (((int64_t)b * D + t) * Hv + h) * dk
                                       : g + ((int64_t)b * D + t) * Hv + h;
                for (int c = 0; c < dk; ++c) alpha[c] = exp(kda ? gt[c] : gt[0]);
                const double bt = beta[((int64_t)b * D + t) * Hv + h];
                delta_rule_token_d(S + (int64_t)h * dv * dk, dk, dv, qn, kn, vr, alpha, bt, scale,
                                   o, dd);
                for (int i = 0; i < dv; ++i) ob[(int64_t)h * dv + i] = orc_round(o[i], io_dtype);
                for (int i = 0; i < dv; ++i) {
                    ring_d[ring_at(slot, Hv, L, h, pos, dv) + i] = orc_round(dd[i], io_dtype);
                    ring_rawv[ring_at(slot, Hv, L, h, pos, dv) + i] = vr[i];
                }
                for (int c = 0; c < dk; ++c) {
                    ring_k[ring_at(slot, Hv, L, h, pos, dk) + c] = orc_round(kn[c], io_dtype);
                    ring_rawk[ring_at(slot, Hv, L, h, pos, dk) + c] = kr[c];
                }
                if (kda)
                    for (int c = 0; c < dk; ++c) ring_g[ring_at(slot, Hv, L, h, pos, dk) + c] = gt[c];
                else
                    ring_g[ring_at(slot, Hv, L, h, pos, 1)] = gt[0];
                ring_beta[ring_at(slot, Hv, L, h, pos, 1)] = bt;
            }
        }
    }
    free(S); free(hist); free(y); free(qn); free(kn); free(alpha); free(o); free(dd);
    return 0;
}

/* Exact commit: for each request, the first accepted[b] ring steps (from
 * position ring_base[b]) are replayed in fp64 from the state of pool row
 * slots[b], which is then stored back rounded to state_dtype. */
int orc_commit(int kda, int B, const int32_t *accepted, int Hv, int dk, int dv,
               const int32_t *slots, double *ssm_pool, int64_t ssm_stride, int state_dtype,
               int L, const int32_t *ring_base, const double *ring_g, const double *ring_rawv,
               const double *ring_rawk, const double *ring_beta, double eps)
{
    const size_t state_elems = (size_t)Hv * dv * dk;
    double *kn = malloc(sizeof(double) * dk), *alpha = malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        const int slot = slots[b];
        double *S = ssm_pool + (int64_t)slot * ssm_stride;
        for (int t = 0; t < accepted[b]; ++t) {
            const int pos = (ring_base[b] + t) & (L - 1);
            for (int h = 0; h < Hv; ++h) {
                l2norm(ring_rawk + ring_at(slot, Hv, L, h, pos, dk), kn, dk, eps);
                for (int c = 0; c < dk; ++c)
                    alpha[c] = exp(kda ? ring_g[ring_at(slot, Hv, L, h, pos, dk) + c]
                                       : ring_g[ring_at(slot, Hv, L, h, pos, 1)]);
                delta_rule_token_d(S + (int64_t)h * dv * dk, dk, dv, NULL, kn,
                                   ring_rawv + ring_at(slot, Hv, L, h, pos, dv), alpha,
                                   ring_beta[ring_at(slot, Hv, L, h, pos, 1)], 0.0, NULL, NULL);
            }
        }
        for (size_t i = 0; i < state_elems; ++i) S[i] = orc_round(S[i], state_dtype);
    }
    free(kn); free(alpha);
    return 0;
}

/* ReplaySSM fast rebuild ([mamba-ish] ReplaySSM "d / k / g" passage): the
 * state after m ring steps is the checkpoint decayed by the product of the
 * steps' alphas plus every step's rank-1 term d_j k_j^T decayed by the alphas
 * of the steps after it,
 *     S_m = S_0 Diag(prod_{i<=m} alpha_i)
 *           + sum_{j<=m} d_j (k_j . prod_{j<i<=m} alpha_i)^T,   alpha = exp(g),
 * with no per-step state and no replay of the delta rule (d is read from the
 * ring).  For each request the checkpoint is pool row slots[b]; the m[b] steps
 * start at ring position ring_base[b]; S_m is stored to row dst[b] (rounded to
 * state_dtype).  With q [B, Hv, dk] (raw; L2-normalised here, as in decode),
 * out [B, Hv, dv] = scale S_m q_hat, rounded to io_dtype. */
int orc_ring_fold(int kda, int B, const int32_t *m, int Hv, int dk, int dv,
                  const int32_t *slots, const int32_t *dst, double *ssm_pool,
                  int64_t ssm_stride, int state_dtype, int L, const int32_t *ring_base,
                  const double *ring_d, const double *ring_k, const double *ring_g,
                  const double *q, double *out, int io_dtype, double eps, double scale)
{
    const size_t head = (size_t)dv * dk;
    double *S = malloc(sizeof(double) * head);
    double *decay = malloc(sizeof(double) * dk), *qn = malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        const int slot = slots[b];
        for (int h = 0; h < Hv; ++h) {
            const double *S0 = ssm_pool + (int64_t)slot * ssm_stride + (int64_t)h * head;
            /* checkpoint term: S_0 Diag(prod of all m alphas) */
            for (int c = 0; c < dk; ++c) decay[c] = 1.0;
            for (int i = 0; i < m[b]; ++i) {
                const int pos = (ring_base[b] + i) & (L - 1);
                for (int c = 0; c < dk; ++c)
                    decay[c] *= exp(kda ? ring_g[ring_at(slot, Hv, L, h, pos, dk) + c]
                                        : ring_g[ring_at(slot, Hv, L, h, pos, 1)]);
            }
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c) S[(int64_t)r * dk + c] = S0[(int64_t)r * dk + c] * decay[c];
            /* rank-1 terms, each decayed by the steps after it */
            for (int j = 0; j < m[b]; ++j) {
                const int pj = (ring_base[b] + j) & (L - 1);
                for (int c = 0; c < dk; ++c) decay[c] = 1.0;
                for (int i = j + 1; i < m[b]; ++i) {
                    const int pos = (ring_base[b] + i) & (L - 1);
                    for (int c = 0; c < dk; ++c)
                        decay[c] *= exp(kda ? ring_g[ring_at(slot, Hv, L, h, pos, dk) + c]
                                            : ring_g[ring_at(slot, Hv, L, h, pos, 1)]);
                }
                const double *dj = ring_d + ring_at(slot, Hv, L, h, pj, dv);
                const double *kj = ring_k + ring_at(slot, Hv, L, h, pj, dk);
                for (int r = 0; r < dv; ++r)
                    for (int c = 0; c < dk; ++c) S[(int64_t)r * dk + c] += dj[r] * kj[c] * decay[c];
            }
            if (q && out) {
                l2norm(q + ((int64_t)b * Hv + h) * dk, qn, dk, eps);
                for (int r = 0; r < dv; ++r) {
                    double p = 0.0;
                    for (int c = 0; c < dk; ++c) p += S[(int64_t)r * dk + c] * qn[c];
                    out[((int64_t)b * Hv + h) * dv + r] = orc_round(scale * p, io_dtype);
                }
            }
            double *Sd = ssm_pool + (int64_t)dst[b] * ssm_stride + (int64_t)h * head;
            for (size_t i = 0; i < head; ++i) Sd[i] = orc_round(S[i], state_dtype);
        }
    }
    free(S); free(decay); free(qn);
    return 0;
}
