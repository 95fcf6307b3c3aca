/*
 * la.h -- C ABI of libla: the recurrent-state path of hybrid linear-attention
 * layers (Kimi Delta Attention and Gated DeltaNet) on AMD MI355X (gfx950).
 *
 * The method.  Per request and value head, a fixed-size state S[d_v, d_k]
 * (row i = value channel i, d_k contiguous) advances once per token:
 *     S' = S Diag(alpha),  d = beta (v - S' k),  S = S' + d k^T,  o = scale S q
 * with alpha = exp(g).  KDA has one log-decay g per key channel; GDN has one
 * scalar per value head.  q and k are L2-normalised, x / sqrt(|x|^2 + eps).
 * Gates.  Every call takes any g <= 0, including g = -inf: a full reset of
 * those channels at that token (exp(-inf) = 0).  The chunked prefill forms
 * the same result as the token-by-token rule over that whole range (no
 * regime bound): a full reset of every key channel starts a new segment of
 * its decay bookkeeping, and 16-token blocks whose decay is too strong for
 * a factorised product form their decay factors element by element.
 * Sources: the decode kernel's steps and the in-place slot update in
 * "SGLang之KV Cache内存池机制" (yuyanqi.com) section 8.5; the state and conv
 * pool layouts in its section 8.2; the per-key-channel alpha of KDA and the
 * exact replay (normalise k, decay, residual times beta, rank-1 update) in the
 * ReplaySSM passages of xxmr.cn/news/181459; the short conv in that page's
 * "Conv state" passage and in hotelren.com/news/5417338 section 2.1.
 *
 * Short conv.  A depthwise causal convolution of kernel 4 over the projected
 * q|k|v channels x[C], C = 2 H_qk d_k + H_v d_v, channel blocks
 * [Q heads | K heads | V heads], head-major inside each block.  With the
 * 3-token history h[0..2] (row 0 oldest) kept per slot:
 *     y[c] = SiLU( w[c,0] h[0][c] + w[c,1] h[1][c] + w[c,2] h[2][c]
 *                  + w[c,3] x[c] + bias[c] )
 * then the history rolls: h <- [h[1], h[2], x].
 *
 * Conventions shared by every call.
 *   - Device pointers unless stated; every buffer is owned by the caller.
 *     The library never allocates, frees or synchronises: each call only
 *     launches kernels on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns.
 *   - Dtype codes: LA_F32 or LA_BF16.  Weights (w, bias), gates (g, beta)
 *     are always fp32; slots and cu_seqlens are int32.
 *   - Pools have `num_rows` = P + 1 rows; row 0 is the padding row (several
 *     padded entries may name it; its contents are then undefined).  A pool
 *     row is addressed as base + slot * slot_stride (elements), so per-layer
 *     views of a [layers, P+1, ...] tensor work.  Inner dims are contiguous.
 *   - Pools are read and written in place, only at the rows named by the
 *     slots.  Non-zero slots that a call writes must be distinct (else the
 *     result is undefined).  Prefill calls read slot_in and write slot_out:
 *     slot_in values may repeat (a row only read) and slot_in[n] ==
 *     slot_out[n] is allowed, but no sequence may read (slot_in >= 1) a row
 *     that another sequence writes.  Slots outside [0, num_rows) are skipped
 *     by the kernels (their outputs are written as zeros and no pool row is
 *     touched); with the environment variable LA_CHECK=1 the call instead
 *     copies the slots to the host, synchronously, and returns LA_ERR_SLOT
 *     for a slot out of range or a breach of these rules.
 *   - Alignment: every pointer must be 16-byte aligned and every row stride
 *     a multiple of 16 bytes (LA_ERR_ARG otherwise).
 *   - A prefill call with no tokens (T == 0) reads none of its per-token
 *     buffers (q, k, v, x, g, beta, out, y), which may then be NULL; it still
 *     hands each sequence's state (and conv history) from slot_in to
 *     slot_out.
 *   - Errors: no exception crosses the ABI.  Calls return an LA_* status;
 *     la_last_error() gives a thread-local message for the last failure.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_VERSION 1

/* Status codes. */
#define LA_OK 0
#define LA_ERR_ARG (-1)         /* null pointer, bad dimension, misalignment */
#define LA_ERR_UNSUPPORTED (-2) /* dtype combination or head dim not built */
#define LA_ERR_WORKSPACE (-3)   /* workspace missing or too small */
#define LA_ERR_SLOT (-4)        /* LA_CHECK=1 only: bad or duplicate slot */
#define LA_ERR_HIP (-5)         /* a HIP call or kernel launch failed */

/* Dtype codes. */
#define LA_F32 0
#define LA_BF16 1

/* Prefill precision modes (kda_prefill_chunked / gdn_prefill_chunked): the
 * operand precision of the matrix-core products.  Accumulation is fp32 in
 * both, and the state carried between blocks is fp32; both meet a 1e-4
 * relative error on fp32 states. */
#define LA_PREFILL_FP32 0   /* fp32 operands (v_mfma_f32_16x16x4f32) */
#define LA_PREFILL_BF16X3 1 /* two-term bf16 split of each operand, three bf16
                               products (about 2^-16 relative per product) */

int la_version(void);

/* Thread-local text of the last error raised on this thread ("" if none). */
const char *la_last_error(void);

/* Host call.  Bytes of the conv and SSM state pools for `layers` layers and
 * `slots` usable slots (slots + 1 rows each, row 0 = padding), the sizes the
 * allocation logs print (hotelren.com/news/5417338 section 4.2; the ReplaySSM
 * allocation log of xxmr.cn/news/181459):
 *   ssm  = layers (slots+1) H_v d_v d_k  size(state_dtype)
 *   conv = layers (slots+1) 3 C          size(conv_dtype)
 * (section 8.2 of the pool page gives the [layers, pool_size+1, ...] shapes;
 * the allocation logs of hotelren.com section 4.2 follow from it).
 * Returns LA_OK, or LA_ERR_ARG for a negative size or unknown dtype. */
int la_pool_bytes(int layers, int slots, int H_v, int d_v, int d_k, int conv_channels,
                  int state_dtype, int conv_dtype, int64_t *ssm_bytes, int64_t *conv_bytes);

/* Host call.  Bytes of each buffer of the ReplaySSM ring (la_ring below) for
 * `layers` layers, `slots` usable slots (slots + 1 rows, as the pools),
 * H_v value heads and L positions: d_bytes for d and for rawv
 * ([rows, H_v, L, d_v] in io_dtype), k_bytes for k and for rawk
 * ([rows, H_v, L, d_k] in io_dtype), g_bytes for g (fp32, [rows, H_v, L,
 * d_k] with kda != 0, else [rows, H_v, L]) and beta_bytes for beta (fp32,
 * [rows, H_v, L]).  Source: the ring shapes [69, 120, 12, 16, 128] and the
 * "ring buffers allocated (L16)" log of the ReplaySSM passage of
 * xxmr.cn/news/181459.  Any output pointer may be NULL.  Returns LA_OK, or
 * LA_ERR_ARG for a negative size or unknown dtype. */
int la_ring_bytes(int layers, int slots, int H_v, int L, int d_k, int d_v, int io_dtype, int kda,
                  int64_t *d_bytes, int64_t *k_bytes, int64_t *g_bytes, int64_t *beta_bytes);

/* One decode token of the short conv + SiLU, standalone.  Source: the
 * causal_conv1d_update step of forward_decode in "SGLang之KV Cache内存池机制"
 * section 8.5 (in place on the conv pool rows named by the cache indices) and
 * the "Conv state" passage of xxmr.cn/news/181459 (a 3-token history per
 * request).
 *   x [B, C] (x_dtype) input projections of the current token;
 *   w [C, 4], bias [C] or NULL;
 *   conv_pool rows [3, C] (conv_dtype) at conv_pool + slot * conv_slot_stride;
 *   slots [B]; y [B, C] (x_dtype) receives the activations.
 * Rolls the history of each named row in place (the current input becomes
 * row 2, converted to conv_dtype; a bit copy when the dtypes agree). */
int shortconv_update(int B, int C, const void *x, int x_dtype, const float *w,
                     const float *bias, void *conv_pool, int64_t conv_slot_stride,
                     int conv_dtype, int num_rows, const int32_t *slots, void *y,
                     void *stream);

/* One KDA decode token per request, fused: short conv + SiLU over x, split
 * into q [H_qk, d_k] | k [H_qk, d_k] | v [H_v, d_v], L2 norm of q and k, then
 * the gated delta rule with a per-key-channel decay, in place on the state.
 * Source: forward_decode in "SGLang之KV Cache内存池机制" section 8.5 (conv
 * update, then the recurrence reading and writing the state pool rows in
 * place: h *= exp(g), the delta correction, h += k v, o = h q) and the "KDA
 * recurrent update" passage of xxmr.cn/news/181459 (alpha per key channel).
 *   x [B, C] (io_dtype); C = 2 H_qk d_k + H_v d_v.
 *   conv_w [C, 4] or NULL: NULL means x already holds the post-conv q|k|v;
 *     the conv, the SiLU and the conv pool are then skipped (conv_pool may be
 *     NULL).  conv_b [C] or NULL.
 *   conv_pool rows [3, C] (conv_dtype), see shortconv_update.
 *   g [B, H_v, d_k] fp32 log-decays (alpha = exp(g)); beta [B, H_v] fp32.
 *   slots [B]; ssm_pool rows [H_v, d_v, d_k] (state_dtype) at
 *     ssm_pool + slot * ssm_slot_stride.
 *   out [B, H_v, d_v] (io_dtype) = scale * S_t q_t with the updated state.
 *   eps: L2-norm epsilon (1e-6 in the reference workloads); scale: output
 *   scale (1.0).
 * Supported: d_k == d_v in {16, 32, 64, 128}; H_v a multiple of H_qk (value
 * head h reads q/k head h / (H_v / H_qk)); every dtype pair of fp32/bf16.
 * Arithmetic is fp32; bf16 stores round to nearest even. */
int kda_decode_step(int B, int H_qk, int H_v, int d_k, int d_v, const void *x, int io_dtype,
                    const float *conv_w, const float *conv_b, void *conv_pool,
                    int64_t conv_slot_stride, int conv_dtype, const float *g,
                    const float *beta, const int32_t *slots, int num_rows, void *ssm_pool,
                    int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                    float scale, void *stream);

/* GDN decode: as kda_decode_step with one log-decay per value head,
 * g [B, H_v] fp32 (the decay Diag(alpha) is alpha I).  Source: the "KDA
 * recurrent update" passage of xxmr.cn/news/181459, which sets KDA's
 * per-key-channel alpha against the one scalar per head of the other linear
 * layers, and the forward_decode steps of "SGLang之KV Cache内存池机制"
 * section 8.5. */
int gdn_decode_step(int B, int H_qk, int H_v, int d_k, int d_v, const void *x, int io_dtype,
                    const float *conv_w, const float *conv_b, void *conv_pool,
                    int64_t conv_slot_stride, int conv_dtype, const float *g,
                    const float *beta, const int32_t *slots, int num_rows, void *ssm_pool,
                    int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                    float scale, void *stream);

/* Short conv + SiLU over N packed sequences (prefill).  Source: the conv of
 * forward_extend in "SGLang之KV Cache内存池机制" section 8.5 (varlen over
 * cu_seqlens, history read from and written back to each request's slot).
 * Sequence n covers
 * tokens [cu_seqlens[n], cu_seqlens[n+1]) of x [T, C] (io_dtype); its history
 * comes from conv-pool row slot_in[n] (zeros when slot_in[n] < 0) and the last
 * three pre-conv inputs (older history shifted in when the sequence is
 * shorter than three tokens) are written to row slot_out[n] (slot_in[n] ==
 * slot_out[n] is allowed).  y [T, C] (io_dtype) receives the activations.
 * cu_seqlens [N+1] must be non-decreasing from 0 to T. */
int shortconv_prefill(int N, int T, int C, const void *x, int io_dtype,
                      const int32_t *cu_seqlens, const int32_t *slot_in,
                      const int32_t *slot_out, const float *w, const float *bias,
                      void *conv_pool, int64_t conv_slot_stride, int conv_dtype,
                      int num_rows, void *y, void *stream);

/* Chunked KDA prefill over N packed sequences (extend: the initial state is
 * read from the pool, the final state written back; the result is that of
 * the token-by-token recurrence, computed by blocks of 64 tokens).  Source:
 * forward_extend in "SGLang之KV Cache内存池机制" section 8.5 (chunk size 64,
 * inter-chunk recurrence plus intra-chunk parallel work, state read from and
 * written to the pool by cache index) and the unrolled sum of the ReplaySSM
 * fast-rebuild passage of xxmr.cn/news/181459 (the block algebra).
 *   q [T, H_qk, d_k], k [T, H_qk, d_k], v [T, H_v, d_v] (io_dtype; raw,
 *     post-conv: q and k are L2-normalised inside) with token strides
 *     q_stride, k_stride, v_stride in elements (>= the row size; lets q|k|v be
 *     views into one [T, C] conv output).
 *   g [T, H_v, d_k] fp32; beta [T, H_v] fp32; cu_seqlens [N+1].
 *   slot_in [N] (< 0: zero initial state), slot_out [N] rows of
 *     ssm_pool [H_v, d_v, d_k] (state_dtype).
 *   out [T, H_v, d_v] (io_dtype).
 *   mode: LA_PREFILL_FP32 or LA_PREFILL_BF16X3.
 *   workspace: device scratch of at least kda_prefill_workspace_bytes(...)
 *     bytes, 256-byte aligned; contents need no initialisation.
 * Supported: d_k == d_v == 128; H_v a multiple of H_qk; H_v <= 4096 (larger
 * values return LA_ERR_UNSUPPORTED: a 64-token block's outputs are addressed
 * with 32-bit offsets). */
int kda_prefill_chunked(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                        int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                        int64_t v_stride, int io_dtype, const float *g, const float *beta,
                        const int32_t *cu_seqlens, const int32_t *slot_in,
                        const int32_t *slot_out, int num_rows, void *ssm_pool,
                        int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                        float scale, int mode, void *workspace, size_t workspace_bytes,
                        void *stream);

/* GDN prefill: as kda_prefill_chunked with g [T, H_v] (one log-decay per
 * value head) and a workspace of gdn_prefill_workspace_bytes(...).  Source:
 * forward_extend in "SGLang之KV Cache内存池机制" section 8.5. */
int gdn_prefill_chunked(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                        int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                        int64_t v_stride, int io_dtype, const float *g, const float *beta,
                        const int32_t *cu_seqlens, const int32_t *slot_in,
                        const int32_t *slot_out, int num_rows, void *ssm_pool,
                        int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                        float scale, int mode, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Chunked prefill with the short conv fused into its loads.  The extend path
 * of "SGLang之KV Cache内存池机制" (yuyanqi.com) section 8.5 hands the chunked
 * kernel the mixed q|k|v projections of a varlen batch, with the conv and SSM
 * state of each request in the same pool slot; here the conv + SiLU of
 * shortconv_prefill runs inside the prefill's loads instead of as a pass of
 * its own (no [T, C] conv output is written or read back).
 *   x [T, C] (io_dtype) pre-conv projections, C = 2 H_qk d_k + H_v d_v,
 *     channel blocks [Q heads | K heads | V heads] as in kda_decode_step.
 *   conv_w [C, 4], conv_b [C] or NULL; conv_pool rows [3, C] (conv_dtype)
 *     at conv_pool + slot * conv_slot_stride, indexed by the same slot_in /
 *     slot_out as ssm_pool: the history comes from slot_in (zeros when < 0)
 *     and the last three pre-conv inputs go to slot_out, as in
 *     shortconv_prefill (slot_in == slot_out is allowed).
 *   Every other argument is that of kda_prefill_chunked.
 * The conv activations stay fp32 between the conv and the prefill (the
 * standalone pair rounds them to io_dtype in between).  Sequences whose
 * slots are out of range get zero outputs and touch neither pool. */
int kda_prefill_conv(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *x,
                     int io_dtype, const float *conv_w, const float *conv_b, void *conv_pool,
                     int64_t conv_slot_stride, int conv_dtype, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const int32_t *slot_in,
                     const int32_t *slot_out, int num_rows, void *ssm_pool,
                     int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                     float scale, int mode, void *workspace, size_t workspace_bytes,
                     void *stream);

/* GDN form of kda_prefill_conv: g [T, H_v]. */
int gdn_prefill_conv(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *x,
                     int io_dtype, const float *conv_w, const float *conv_b, void *conv_pool,
                     int64_t conv_slot_stride, int conv_dtype, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const int32_t *slot_in,
                     const int32_t *slot_out, int num_rows, void *ssm_pool,
                     int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                     float scale, int mode, void *workspace, size_t workspace_bytes,
                     void *stream);

/* kda_prefill_chunked without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a 128 MiB device
 * array inside the library, one per GPU, held from this call's first use on
 * that GPU until the process ends; its address is looked up once per device
 * (the current device must be the stream's).  Arguments, layouts and results
 * are those of kda_prefill_chunked.  The call allocates and frees nothing;
 * LA_CHECK=1 does not apply to it (its host copies would allocate).
 * Returns LA_ERR_WORKSPACE when kda_prefill_workspace_bytes(...) exceeds
 * 128 MiB (about 47,000 token x value-head pairs; 3,900 tokens at 12
 * heads).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised. */
int kda_prefill_chunked_noalloc(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                                int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                                int64_t v_stride, int io_dtype, const float *g,
                                const float *beta, const int32_t *cu_seqlens,
                                const int32_t *slot_in, const int32_t *slot_out, int num_rows,
                                void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
                                void *out, float eps, float scale, int mode, void *stream);

/* Host calls: workspace bytes kda_prefill_chunked / kda_prefill_conv and
 * gdn_prefill_chunked / gdn_prefill_conv need for N sequences and T tokens
 * (0 for invalid arguments).  The workspace holds the per-block quantities
 * the inter-block chain reads (the intra-chunk part of forward_extend in
 * "SGLang之KV Cache内存池机制" section 8.5). */
size_t kda_prefill_workspace_bytes(int N, int T, int H_qk, int H_v, int d_k, int d_v, int mode);
size_t gdn_prefill_workspace_bytes(int N, int T, int H_qk, int H_v, int d_k, int d_v, int mode);

/* ---- Speculative decode (multi-token verify with an exact commit) --------
 * Sources: the ReplaySSM passages of xxmr.cn/news/181459 (verify computes
 * every draft step's output from the checkpoint without writing the state
 * back; a per-slot ring records each step; the commit replays the accepted
 * prefix from the checkpoint), its "intermediate_conv_window" passage (the
 * per-step conv history, scattered at the last accepted step) and its
 * state-tracking passage (masked copy of conv + SSM rows to a tracking slot).
 *
 * The ring of step records, one per pool row (slot), value head and step
 * position (L positions, L a power of two; the pages size it as the next
 * power of two >= 2 x the draft tokens of a call).  Step t of request b of a
 * verify call is stored at position (ring_base[b] + t) mod L.  Vectors are in
 * the call's I/O dtype; gates are fp32.  All pointers are device pointers,
 * owned by the caller; the struct itself is read on the host.
 *   d     [num_rows, H_v, L, d_v]  beta (rawv - S' k): the step's corrected value
 *   k     [num_rows, H_v, L, d_k]  the normalised key
 *   rawv  [num_rows, H_v, L, d_v]  the value entering the delta rule
 *   rawk  [num_rows, H_v, L, d_k]  the key before normalisation
 *   g     [num_rows, H_v, L, d_k] (KDA) or [num_rows, H_v, L] (GDN), fp32
 *   beta  [num_rows, H_v, L] fp32 */
typedef struct la_ring {
    int L;
    void *d, *k, *rawv, *rawk;
    float *g, *beta;
} la_ring;

/* KDA verify: for each request b, the first n_tok[b] (<= D) of its D draft
 * tokens run from the conv history and state of pool row slots[b] -- neither
 * pool is modified -- through the short conv + SiLU (output rounded to
 * io_dtype, the dtype a separate conv kernel would store), the L2 norms and the
 * gated delta rule.  Two forms, chosen by D: up to 8 tokens the chunk form
 * (the outputs and d from one product of the checkpoint with the steps'
 * decayed keys and queries, plus the 8x8 intra-step terms: equal to the
 * sequential rule up to rounding); beyond 8 the sequential form, the state
 * carried in fp32 across the tokens with the commit's per-step arithmetic.
 *   x [B, D, C] (io_dtype); conv_w [C, 4] or NULL (x is then post-conv and
 *     conv_windows is not written); conv_b [C] or NULL.
 *   g [B, D, H_v, d_k] fp32; beta [B, D, H_v] fp32; slots, n_tok [B] int32.
 *   out [B, D, H_v, d_v] (io_dtype): each step's o = scale S_t q_t; zeros for
 *     steps past n_tok[b] and for skipped entries (slot out of range).
 *   conv_windows [B, D, 3, C] (conv_dtype): the conv history after each step
 *     (what the conv pool would hold had that step been the last accepted).
 *   ring / ring_base [B]: each step's record is written to the ring rows of
 *     slots[b] (see la_ring); L >= D is required.
 * Supported: d_k == d_v == 128; H_v a multiple of H_qk; fp32/bf16 dtypes. */
int kda_verify(int B, int D, const int32_t *n_tok, int H_qk, int H_v, int d_k, int d_v,
               const void *x, int io_dtype, const float *conv_w, const float *conv_b,
               const void *conv_pool, int64_t conv_slot_stride, int conv_dtype, const float *g,
               const float *beta, const int32_t *slots, int num_rows, const void *ssm_pool,
               int64_t ssm_slot_stride, int state_dtype, void *out, void *conv_windows,
               const la_ring *ring, const int32_t *ring_base, float eps, float scale,
               void *stream);

/* GDN verify: as kda_verify with g [B, D, H_v] (one log-decay per head). */
int gdn_verify(int B, int D, const int32_t *n_tok, int H_qk, int H_v, int d_k, int d_v,
               const void *x, int io_dtype, const float *conv_w, const float *conv_b,
               const void *conv_pool, int64_t conv_slot_stride, int conv_dtype, const float *g,
               const float *beta, const int32_t *slots, int num_rows, const void *ssm_pool,
               int64_t ssm_slot_stride, int state_dtype, void *out, void *conv_windows,
               const la_ring *ring, const int32_t *ring_base, float eps, float scale,
               void *stream);

/* Exact commit (KDA): for each request, the first accepted[b] (<= L) ring
 * steps from position ring_base[b] are replayed from the state of pool row
 * slots[b] with k = rawk / sqrt(|rawk|^2 + eps), alpha = exp(g),
 * S <- S Diag(alpha), d = beta (rawv - S k), S <- S + d k^T (fp32), and the
 * result is stored back (state_dtype).  accepted[b] = 0 leaves the row
 * untouched.  io_dtype is the dtype of the ring's vectors.  The replay runs
 * the same per-row arithmetic as verify, so committing a verify's first a
 * steps gives the state verify held after step a. */
int kda_commit(int B, const int32_t *accepted, int H_v, int d_k, int d_v, const int32_t *slots,
               int num_rows, void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
               int io_dtype, const la_ring *ring, const int32_t *ring_base, float eps,
               void *stream);

/* Exact commit (GDN): as kda_commit with the ring's per-head g. */
int gdn_commit(int B, const int32_t *accepted, int H_v, int d_k, int d_v, const int32_t *slots,
               int num_rows, void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
               int io_dtype, const la_ring *ring, const int32_t *ring_base, float eps,
               void *stream);

/* Conv-state commit after verify: for every b with mask[b] != 0 (mask NULL =
 * all) and 0 <= step[b] < D, conv pool row slots[b] becomes
 * windows[b, step[b]] (windows [B, D, 3, C] in conv_dtype, as written by
 * *_verify).  3 C elements must be a multiple of 16 bytes. */
int conv_window_scatter(int B, int D, int C, const uint8_t *mask, const int32_t *slots,
                        const int32_t *step, const void *windows, void *conv_pool,
                        int64_t conv_slot_stride, int conv_dtype, int num_rows, void *stream);

/* State tracking: for every b with mask[b] != 0 (mask NULL = all), pool rows
 * dst[b] of the conv pool (conv_row_elems elements of conv_dtype) and of the
 * SSM pool (ssm_row_elems elements of state_dtype) become bit copies of rows
 * src[b].  Rows must be multiples of 16 bytes.  src == dst is a no-op; a dst
 * that is another entry's src gives an undefined result. */
int state_track_copy(int B, const uint8_t *mask, const int32_t *src, const int32_t *dst,
                     void *conv_pool, int64_t conv_slot_stride, int64_t conv_row_elems,
                     int conv_dtype, void *ssm_pool, int64_t ssm_slot_stride,
                     int64_t ssm_row_elems, int state_dtype, int num_rows, void *stream);

/* ReplaySSM fast rebuild (KDA): for each request, the state after the m[b]
 * (<= L) ring steps from position ring_base[b], from the checkpoint in pool
 * row slots[b] and the steps' (d, k, g) alone (no replay of the delta rule):
 *     S_m = S_0 Diag(prod alpha) + sum_j d_j (k_j . prod_{i>j} alpha_i)^T,
 * the unrolled sum of the ReplaySSM d/k/g passage of xxmr.cn/news/181459.
 * S_m is stored to row dst_slots[b] (dst_slots NULL: in place); destination
 * rows must not be another entry's source.  With q [B, H_v, d_k] (raw, L2-
 * normalised inside) and out [B, H_v, d_v], out = scale S_m q_hat.  io_dtype
 * is the dtype of the ring's vectors, q and out.  Supported: d_k == d_v == 128. */
int kda_ring_fold(int B, const int32_t *m, int H_v, int d_k, int d_v, const int32_t *slots,
                  const int32_t *dst_slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                  const void *q, void *out, float eps, float scale, void *stream);

/* Fast rebuild (GDN): as kda_ring_fold with the ring's per-head g. */
int gdn_ring_fold(int B, const int32_t *m, int H_v, int d_k, int d_v, const int32_t *slots,
                  const int32_t *dst_slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                  const void *q, void *out, float eps, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
