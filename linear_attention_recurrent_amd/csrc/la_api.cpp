// la_api.cpp -- the extern "C" entry points declared in include/la.h.
//
// Host side only: argument validation, the optional checked mode (LA_CHECK=1:
// slots and sequence offsets copied to the host and verified), dtype / head
// dim dispatch and error reporting.  Every computation happens in the HIP
// kernels; nothing here allocates, frees or synchronises outside checked mode
// (the error text lives in a fixed thread-local buffer).  The one device
// object defined here is the scratch array of kda_prefill_chunked_noalloc.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "la.h"
#include "la_internal.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = 0;
    return LA_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool checked_mode()
{
    const char *s = std::getenv("LA_CHECK");
    return s && s[0] == '1';
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d == LA_F32 || d == LA_BF16; }

int dsize(int d) { return d == LA_BF16 ? 2 : 4; }

bool supported_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Copies n int32 values from device to host (checked mode only).
int fetch_i32(const int32_t *dev, int n, std::vector<int32_t> &host, hipStream_t stream)
{
    host.resize(n);
    if (n == 0) return LA_OK;
    hipError_t e = hipMemcpyAsync(host.data(), dev, sizeof(int32_t) * n, hipMemcpyDeviceToHost,
                                  stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return hip_status(e, "checked mode: copying indices to the host");
}

// Non-zero slots in [1, num_rows) must be distinct; `allow_negative` admits
// negative entries (prefill slot_in: fresh sequence).
int check_slots(const std::vector<int32_t> &s, int num_rows, bool allow_negative, const char *name)
{
    std::unordered_set<int32_t> seen;
    for (size_t i = 0; i < s.size(); ++i) {
        const int32_t v = s[i];
        if (v < 0 && allow_negative) continue;
        if (v < 0 || v >= num_rows)
            return fail(LA_ERR_SLOT, "%s[%zu] = %d outside [0, %d)", name, i, v, num_rows);
        if (v != 0 && !seen.insert(v).second)
            return fail(LA_ERR_SLOT, "%s[%zu] = %d repeats a slot of this call", name, i, v);
    }
    return LA_OK;
}

// Prefill slots: slot_out entries in [0, num_rows), non-zero ones distinct;
// slot_in entries < 0 (fresh) or in [0, num_rows), repeats allowed (a row
// only read); and no sequence may read (slot_in >= 1) a row that another
// sequence writes (its slot_out), since the write of one workgroup would race
// the read of another.  slot_in[n] == slot_out[n] is the in-place default.
int check_prefill_slots(const std::vector<int32_t> &si, const std::vector<int32_t> &so,
                        int num_rows)
{
    std::unordered_map<int32_t, size_t> writer;
    for (size_t m = 0; m < so.size(); ++m) {
        const int32_t v = so[m];
        if (v < 0 || v >= num_rows)
            return fail(LA_ERR_SLOT, "slot_out[%zu] = %d outside [0, %d)", m, v, num_rows);
        if (v != 0 && !writer.emplace(v, m).second)
            return fail(LA_ERR_SLOT, "slot_out[%zu] = %d repeats a slot of this call", m, v);
    }
    for (size_t n = 0; n < si.size(); ++n) {
        const int32_t v = si[n];
        if (v >= num_rows)
            return fail(LA_ERR_SLOT, "slot_in[%zu] = %d outside [0, %d)", n, v, num_rows);
        if (v < 1) continue;
        const auto it = writer.find(v);
        if (it != writer.end() && it->second != n)
            return fail(LA_ERR_SLOT, "slot_in[%zu] = %d is slot_out[%zu] of another sequence", n,
                        v, it->second);
    }
    return LA_OK;
}

int check_cu(const std::vector<int32_t> &cu, int T)
{
    if (cu.empty() || cu[0] != 0 || cu.back() != T)
        return fail(LA_ERR_ARG, "cu_seqlens must start at 0 and end at T = %d", T);
    for (size_t i = 1; i < cu.size(); ++i)
        if (cu[i] < cu[i - 1]) return fail(LA_ERR_ARG, "cu_seqlens decreases at %zu", i);
    return LA_OK;
}

int decode_common(bool kda, int B, int Hqk, int Hv, int dk, int dv, const void *x, int io_dtype,
                  const float *conv_w, const float *conv_b, void *conv_pool,
                  int64_t conv_slot_stride, int conv_dtype, const float *g, const float *beta,
                  const int32_t *slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, void *out, float eps, float scale, void *stream)
{
    const char *fn = kda ? "kda_decode_step" : "gdn_decode_step";
    if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (B >= 0)", fn);
    if (Hv % Hqk != 0)
        return fail(LA_ERR_ARG, "%s: H_v = %d is not a multiple of H_qk = %d", fn, Hv, Hqk);
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype) || !valid_dtype(conv_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if (dk != dv || !supported_head_dim(dk))
        return fail(LA_ERR_UNSUPPORTED, "%s: needs d_k == d_v in {16, 32, 64, 128} (got %d, %d)",
                    fn, dk, dv);
    if (B == 0) return ok();
    if (!x || !g || !beta || !slots || !ssm_pool || !out || (conv_w && !conv_pool))
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {x, g, beta, slots, ssm_pool, out, conv_w, conv_b, conv_pool};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    const int C = 2 * Hqk * dk + Hv * dv;
    if (ssm_slot_stride < (int64_t)Hv * dv * dk || (ssm_slot_stride * dsize(state_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: ssm_slot_stride %lld must be >= H_v d_v d_k and a multiple "
                    "of 16 bytes", fn, (long long)ssm_slot_stride);
    if (conv_w && (conv_slot_stride < 3LL * C || (conv_slot_stride * dsize(conv_dtype)) % 16))
        return fail(LA_ERR_ARG, "%s: conv_slot_stride %lld must be >= 3 C and a multiple of 16 "
                    "bytes", fn, (long long)conv_slot_stride);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "slots")) return rc;
    }
    la::DecodeArgs a{};
    a.B = B; a.Hqk = Hqk; a.Hv = Hv; a.G = Hv / Hqk; a.C = C;
    a.x = x; a.io_dtype = io_dtype;
    a.w = conv_w; a.bias = conv_b;
    a.conv_pool = conv_pool; a.conv_stride = conv_slot_stride; a.conv_dtype = conv_dtype;
    a.g = g; a.beta = beta; a.slots = slots; a.num_rows = num_rows;
    a.ssm_pool = ssm_pool; a.ssm_stride = ssm_slot_stride;
    a.out = out; a.eps = eps; a.scale = scale;
    return hip_status(la::launch_decode(a, dk, state_dtype, kda, st), fn);
}

// The fused short conv of kda_prefill_conv / gdn_prefill_conv.
struct ConvIn {
    const void *x;
    const float *w, *bias;
    void *pool;
    int64_t stride;
    int dtype;
};

// cv == nullptr: q, k, v are the post-conv inputs; otherwise they are unused
// and the conv runs on cv->x inside the prefill.
int prefill_common(bool kda, int N, int T, int Hqk, int Hv, int dk, int dv, const void *q,
                   int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                   int64_t v_stride, int io_dtype, const float *g, const float *beta,
                   const int32_t *cu_seqlens, const int32_t *slot_in, const int32_t *slot_out,
                   int num_rows, void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
                   void *out, float eps, float scale, int mode, void *workspace,
                   size_t workspace_bytes, void *stream, const ConvIn *cv = nullptr,
                   bool may_check = true)
{
    const char *fn = cv ? (kda ? "kda_prefill_conv" : "gdn_prefill_conv")
                        : (kda ? "kda_prefill_chunked" : "gdn_prefill_chunked");
    const int64_t C = 2LL * Hqk * dk + (int64_t)Hv * dv;
    if (cv) {
        q = k = v = cv->x;
        q_stride = k_stride = v_stride = C;
    }
    if (N < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (N, T >= 0)", fn);
    if (Hv % Hqk != 0)
        return fail(LA_ERR_ARG, "%s: H_v = %d is not a multiple of H_qk = %d", fn, Hv, Hqk);
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if (mode != LA_PREFILL_FP32 && mode != LA_PREFILL_BF16X3)
        return fail(LA_ERR_UNSUPPORTED, "%s: unknown precision mode %d", fn, mode);
    if (dk != 128 || dv != 128)
        return fail(LA_ERR_UNSUPPORTED, "%s: needs d_k == d_v == 128 (got %d, %d)", fn, dk, dv);
    if (Hv > 4096)  // a block's outputs are addressed with 32-bit byte offsets
        return fail(LA_ERR_UNSUPPORTED, "%s: H_v = %d exceeds 4096", fn, Hv);
    if (N == 0) return ok();
    // with no tokens the per-token buffers are not read and may be NULL
    if (!cu_seqlens || !slot_in || !slot_out || !ssm_pool ||
        (T > 0 && (!q || !k || !v || !g || !beta || !out)))
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (q_stride < (int64_t)Hqk * dk || k_stride < (int64_t)Hqk * dk || v_stride < (int64_t)Hv * dv ||
        (q_stride * dsize(io_dtype)) % 16 || (k_stride * dsize(io_dtype)) % 16 ||
        (v_stride * dsize(io_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: token strides must cover a token's heads and be multiples "
                    "of 16 bytes", fn);
    if (ssm_slot_stride < (int64_t)Hv * dv * dk || (ssm_slot_stride * dsize(state_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: ssm_slot_stride %lld too small or misaligned", fn,
                    (long long)ssm_slot_stride);
    if (cv) {
        if (!valid_dtype(cv->dtype))
            return fail(LA_ERR_UNSUPPORTED, "%s: conv_dtype must be LA_F32 or LA_BF16", fn);
        if (!cv->w || !cv->pool) return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
        const void *cptrs[] = {cv->w, cv->bias, cv->pool};
        for (const void *p : cptrs)
            if (p && !aligned16(p))
                return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
        if (cv->stride < 3 * C)
            return fail(LA_ERR_ARG, "%s: conv_slot_stride must be >= 3 C = %lld", fn,
                        (long long)(3 * C));
    }
    const size_t need = la::prefill_ws_bytes(N, T, Hqk, Hv, dk, mode);
    if (need && (!workspace || workspace_bytes < need ||
                 (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return fail(LA_ERR_WORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                    fn, need, workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (may_check && checked_mode()) {
        std::vector<int32_t> cu, si, so;
        if (int rc = fetch_i32(cu_seqlens, N + 1, cu, st)) return rc;
        if (int rc = check_cu(cu, T)) return rc;
        if (int rc = fetch_i32(slot_in, N, si, st)) return rc;
        if (int rc = fetch_i32(slot_out, N, so, st)) return rc;
        if (int rc = check_prefill_slots(si, so, num_rows)) return rc;
    }
    la::PrefillArgs a{};
    a.N = N; a.T = T; a.Hqk = Hqk; a.Hv = Hv; a.G = Hv / Hqk; a.D = dk;
    a.q = q; a.k = k; a.v = v;
    a.q_stride = q_stride; a.k_stride = k_stride; a.v_stride = v_stride;
    a.io_dtype = io_dtype; a.g = g; a.beta = beta;
    a.cu = cu_seqlens; a.slot_in = slot_in; a.slot_out = slot_out; a.num_rows = num_rows;
    a.ssm_pool = ssm_pool; a.ssm_stride = ssm_slot_stride; a.state_dtype = state_dtype;
    a.out = out; a.eps = eps; a.scale = scale; a.mode = mode; a.kda = kda;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    if (!cv) return hip_status(la::launch_prefill(a, st), fn);
    a.conv = true; a.x = cv->x; a.C = (int)C; a.w = cv->w; a.bias = cv->bias;
    a.conv_pool = cv->pool; a.conv_stride = cv->stride; a.conv_dtype = cv->dtype;
    if (int rc = hip_status(la::launch_prefill(a, st), fn)) return rc;
    // the hand-off overwrites slot_out's history, so it runs after the
    // prefill has read slot_in's
    la::ConvPrefillArgs c{};
    c.N = N; c.T = T; c.C = (int)C; c.x = cv->x; c.io_dtype = io_dtype;
    c.cu = cu_seqlens; c.slot_in = slot_in; c.slot_out = slot_out; c.w = cv->w;
    c.bias = cv->bias; c.conv_pool = cv->pool; c.conv_stride = cv->stride;
    c.conv_dtype = cv->dtype; c.num_rows = num_rows; c.y = nullptr;
    return hip_status(la::launch_shortconv_handoff(c, st), fn);
}


bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int check_ring(const la_ring *r, int D, const char *fn)
{
    if (!r || !r->d || !r->k || !r->rawv || !r->rawk || !r->g || !r->beta)
        return fail(LA_ERR_ARG, "%s: ring and all of its arrays must be given", fn);
    if (!pow2(r->L) || r->L < D)
        return fail(LA_ERR_ARG, "%s: ring depth L = %d must be a power of two >= %d", fn, r->L, D);
    const void *ptrs[] = {r->d, r->k, r->rawv, r->rawk, r->g, r->beta};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(LA_ERR_ARG, "%s: ring arrays must be 16-byte aligned", fn);
    return LA_OK;
}

la::RingArgs ring_args(const la_ring *r)
{
    la::RingArgs g{};
    g.L = r->L; g.d = r->d; g.k = r->k; g.rawv = r->rawv; g.rawk = r->rawk;
    g.g = r->g; g.beta = r->beta;
    return g;
}

int verify_common(bool kda, int B, int D, const int32_t *n_tok, int Hqk, int Hv, int dk, int dv,
                  const void *x, int io_dtype, const float *conv_w, const float *conv_b,
                  const void *conv_pool, int64_t conv_slot_stride, int conv_dtype,
                  const float *g, const float *beta, const int32_t *slots, int num_rows,
                  const void *ssm_pool, int64_t ssm_slot_stride, int state_dtype, void *out,
                  void *conv_windows, const la_ring *ring, const int32_t *ring_base, float eps,
                  float scale, void *stream)
{
    const char *fn = kda ? "kda_verify" : "gdn_verify";
    if (B < 0 || D <= 0 || Hqk <= 0 || Hv <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (B >= 0)", fn);
    if (Hv % Hqk != 0)
        return fail(LA_ERR_ARG, "%s: H_v = %d is not a multiple of H_qk = %d", fn, Hv, Hqk);
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype) || !valid_dtype(conv_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if (dk != 128 || dv != 128)
        return fail(LA_ERR_UNSUPPORTED, "%s: needs d_k == d_v == 128 (got %d, %d)", fn, dk, dv);
    if (B == 0) return ok();
    if (int rc = check_ring(ring, D, fn)) return rc;
    if (!x || !g || !beta || !slots || !n_tok || !ssm_pool || !out || !ring_base ||
        (conv_w && (!conv_pool || !conv_windows)))
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {x, g, beta, slots, n_tok, ssm_pool, out, ring_base, conv_w, conv_b,
                          conv_pool, conv_windows};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    const int C = 2 * Hqk * dk + Hv * dv;
    if (ssm_slot_stride < (int64_t)Hv * dv * dk || (ssm_slot_stride * dsize(state_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: ssm_slot_stride %lld too small or misaligned", fn,
                    (long long)ssm_slot_stride);
    if (conv_w && (conv_slot_stride < 3LL * C || (conv_slot_stride * dsize(conv_dtype)) % 16))
        return fail(LA_ERR_ARG, "%s: conv_slot_stride %lld too small or misaligned", fn,
                    (long long)conv_slot_stride);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "slots")) return rc;
    }
    la::VerifyArgs a{};
    a.B = B; a.D = D; a.Hqk = Hqk; a.Hv = Hv; a.G = Hv / Hqk; a.C = C; a.n_tok = n_tok;
    a.x = x; a.io_dtype = io_dtype; a.w = conv_w; a.bias = conv_b;
    a.conv_pool = conv_pool; a.conv_stride = conv_slot_stride; a.conv_dtype = conv_dtype;
    a.g = g; a.beta = beta; a.slots = slots; a.num_rows = num_rows;
    a.ssm_pool = ssm_pool; a.ssm_stride = ssm_slot_stride; a.out = out; a.windows = conv_windows;
    a.ring = ring_args(ring); a.ring_base = ring_base; a.eps = eps; a.scale = scale;
    return hip_status(la::launch_verify(a, state_dtype, kda, st), fn);
}

int commit_common(bool kda, int B, const int32_t *accepted, int Hv, int dk, int dv,
                  const int32_t *slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                  float eps, void *stream)
{
    const char *fn = kda ? "kda_commit" : "gdn_commit";
    if (B < 0 || Hv <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (B >= 0)", fn);
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if (dk != 128 || dv != 128)
        return fail(LA_ERR_UNSUPPORTED, "%s: needs d_k == d_v == 128 (got %d, %d)", fn, dk, dv);
    if (B == 0) return ok();
    if (int rc = check_ring(ring, 1, fn)) return rc;
    if (!accepted || !slots || !ssm_pool || !ring_base)
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {accepted, slots, ssm_pool, ring_base};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (ssm_slot_stride < (int64_t)Hv * dv * dk || (ssm_slot_stride * dsize(state_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: ssm_slot_stride %lld too small or misaligned", fn,
                    (long long)ssm_slot_stride);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "slots")) return rc;
    }
    la::CommitArgs a{};
    a.B = B; a.Hv = Hv; a.accepted = accepted; a.slots = slots; a.num_rows = num_rows;
    a.ssm_pool = ssm_pool; a.ssm_stride = ssm_slot_stride; a.io_dtype = io_dtype;
    a.ring = ring_args(ring); a.ring_base = ring_base; a.eps = eps;
    return hip_status(la::launch_commit(a, state_dtype, kda, st), fn);
}


int fold_common(bool kda, int B, const int32_t *m, int Hv, int dk, int dv, const int32_t *slots,
                const int32_t *dst_slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                const void *q, void *out, float eps, float scale, void *stream)
{
    const char *fn = kda ? "kda_ring_fold" : "gdn_ring_fold";
    if (B < 0 || Hv <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (B >= 0)", fn);
    if (!valid_dtype(io_dtype) || !valid_dtype(state_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if (dk != 128 || dv != 128)
        return fail(LA_ERR_UNSUPPORTED, "%s: needs d_k == d_v == 128 (got %d, %d)", fn, dk, dv);
    if (B == 0) return ok();
    if (int rc = check_ring(ring, 1, fn)) return rc;
    if (!m || !slots || !ssm_pool || !ring_base || (!q) != (!out))
        return fail(LA_ERR_ARG, "%s: null pointer argument (q and out go together)", fn);
    const void *ptrs[] = {m, slots, dst_slots, ssm_pool, ring_base, q, out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (ssm_slot_stride < (int64_t)Hv * dv * dk || (ssm_slot_stride * dsize(state_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: ssm_slot_stride %lld too small or misaligned", fn,
                    (long long)ssm_slot_stride);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(dst_slots ? dst_slots : slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "dst_slots")) return rc;
    }
    la::FoldArgs a{};
    a.B = B; a.Hv = Hv; a.m = m; a.slots = slots; a.dst = dst_slots; a.num_rows = num_rows;
    a.ssm_pool = ssm_pool; a.ssm_stride = ssm_slot_stride; a.io_dtype = io_dtype;
    a.ring = ring_args(ring); a.ring_base = ring_base; a.q = q; a.out = out; a.eps = eps;
    a.scale = scale;
    return hip_status(la::launch_fold(a, state_dtype, kda, st), fn);
}

// ---- scratch of kda_prefill_chunked_noalloc --------------------------------
// A file-scope device array stands in for the caller's workspace.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device -- each GPU
// holds its own copy of the array.
constexpr size_t kScratchBytes = size_t(128) << 20;  // 128 MiB per GPU
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's scratch address, or nullptr (after fail()).
void *scratch_address(const char *fn)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        hip_status(e, fn);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        fail(LA_ERR_HIP, "%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(LA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                 hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int la_version(void) { return LA_VERSION; }

const char *la_last_error(void) { return g_err; }

int la_pool_bytes(int layers, int slots, int H_v, int d_v, int d_k, int conv_channels,
                  int state_dtype, int conv_dtype, int64_t *ssm_bytes, int64_t *conv_bytes)
{
    if (layers < 0 || slots < 0 || H_v < 0 || d_v < 0 || d_k < 0 || conv_channels < 0)
        return fail(LA_ERR_ARG, "la_pool_bytes: negative size");
    if (!valid_dtype(state_dtype) || !valid_dtype(conv_dtype))
        return fail(LA_ERR_ARG, "la_pool_bytes: dtype codes must be LA_F32 or LA_BF16");
    const int64_t rows = (int64_t)layers * (slots + 1);
    if (ssm_bytes) *ssm_bytes = rows * H_v * d_v * d_k * dsize(state_dtype);
    if (conv_bytes) *conv_bytes = rows * 3 * conv_channels * dsize(conv_dtype);
    return ok();
}

int shortconv_update(int B, int C, const void *x, int x_dtype, const float *w, const float *bias,
                     void *conv_pool, int64_t conv_slot_stride, int conv_dtype, int num_rows,
                     const int32_t *slots, void *y, void *stream)
{
    if (B < 0 || C <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "shortconv_update: B >= 0, C > 0 and num_rows > 0 required");
    if (!valid_dtype(x_dtype) || !valid_dtype(conv_dtype))
        return fail(LA_ERR_UNSUPPORTED, "shortconv_update: dtype codes must be LA_F32 or LA_BF16");
    if (B == 0) return ok();
    if (!x || !w || !conv_pool || !slots || !y)
        return fail(LA_ERR_ARG, "shortconv_update: null pointer argument");
    const void *ptrs[] = {x, w, bias, conv_pool, slots, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(LA_ERR_ARG, "shortconv_update: pointers must be 16-byte aligned");
    if (conv_slot_stride < 3LL * C)
        return fail(LA_ERR_ARG, "shortconv_update: conv_slot_stride must be >= 3 C");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "slots")) return rc;
    }
    la::ConvStepArgs a{};
    a.B = B; a.C = C; a.x = x; a.x_dtype = x_dtype; a.w = w; a.bias = bias;
    a.conv_pool = conv_pool; a.conv_stride = conv_slot_stride; a.conv_dtype = conv_dtype;
    a.num_rows = num_rows; a.slots = slots; a.y = y;
    return hip_status(la::launch_shortconv_update(a, st), "shortconv_update");
}

int shortconv_prefill(int N, int T, int C, const void *x, int io_dtype, const int32_t *cu_seqlens,
                      const int32_t *slot_in, const int32_t *slot_out, const float *w,
                      const float *bias, void *conv_pool, int64_t conv_slot_stride,
                      int conv_dtype, int num_rows, void *y, void *stream)
{
    if (N < 0 || T < 0 || C <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "shortconv_prefill: N, T >= 0, C > 0, num_rows > 0 required");
    if (!valid_dtype(io_dtype) || !valid_dtype(conv_dtype))
        return fail(LA_ERR_UNSUPPORTED, "shortconv_prefill: dtype codes must be LA_F32 or LA_BF16");
    if (N == 0) return ok();
    if (!cu_seqlens || !slot_in || !slot_out || !w || !conv_pool || (T > 0 && (!x || !y)))
        return fail(LA_ERR_ARG, "shortconv_prefill: null pointer argument");
    const void *ptrs[] = {x, cu_seqlens, slot_in, slot_out, w, bias, conv_pool, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return fail(LA_ERR_ARG, "shortconv_prefill: pointers must be 16-byte aligned");
    if (conv_slot_stride < 3LL * C)
        return fail(LA_ERR_ARG, "shortconv_prefill: conv_slot_stride must be >= 3 C");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> cu, si, so;
        if (int rc = fetch_i32(cu_seqlens, N + 1, cu, st)) return rc;
        if (int rc = check_cu(cu, T)) return rc;
        if (int rc = fetch_i32(slot_in, N, si, st)) return rc;
        if (int rc = fetch_i32(slot_out, N, so, st)) return rc;
        if (int rc = check_prefill_slots(si, so, num_rows)) return rc;
    }
    la::ConvPrefillArgs a{};
    a.N = N; a.T = T; a.C = C; a.x = x; a.io_dtype = io_dtype;
    a.cu = cu_seqlens; a.slot_in = slot_in; a.slot_out = slot_out; a.w = w; a.bias = bias;
    a.conv_pool = conv_pool; a.conv_stride = conv_slot_stride; a.conv_dtype = conv_dtype;
    a.num_rows = num_rows; a.y = y;
    return hip_status(la::launch_shortconv_prefill(a, st), "shortconv_prefill");
}

int kda_decode_step(int B, int H_qk, int H_v, int d_k, int d_v, const void *x, int io_dtype,
                    const float *conv_w, const float *conv_b, void *conv_pool,
                    int64_t conv_slot_stride, int conv_dtype, const float *g, const float *beta,
                    const int32_t *slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                    int state_dtype, void *out, float eps, float scale, void *stream)
{
    return decode_common(true, B, H_qk, H_v, d_k, d_v, x, io_dtype, conv_w, conv_b, conv_pool,
                         conv_slot_stride, conv_dtype, g, beta, slots, num_rows, ssm_pool,
                         ssm_slot_stride, state_dtype, out, eps, scale, stream);
}

int gdn_decode_step(int B, int H_qk, int H_v, int d_k, int d_v, const void *x, int io_dtype,
                    const float *conv_w, const float *conv_b, void *conv_pool,
                    int64_t conv_slot_stride, int conv_dtype, const float *g, const float *beta,
                    const int32_t *slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                    int state_dtype, void *out, float eps, float scale, void *stream)
{
    return decode_common(false, B, H_qk, H_v, d_k, d_v, x, io_dtype, conv_w, conv_b, conv_pool,
                         conv_slot_stride, conv_dtype, g, beta, slots, num_rows, ssm_pool,
                         ssm_slot_stride, state_dtype, out, eps, scale, stream);
}

int kda_prefill_chunked(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                        int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                        int64_t v_stride, int io_dtype, const float *g, const float *beta,
                        const int32_t *cu_seqlens, const int32_t *slot_in,
                        const int32_t *slot_out, int num_rows, void *ssm_pool,
                        int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                        float scale, int mode, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    return prefill_common(true, N, T, H_qk, H_v, d_k, d_v, q, q_stride, k, k_stride, v, v_stride,
                          io_dtype, g, beta, cu_seqlens, slot_in, slot_out, num_rows, ssm_pool,
                          ssm_slot_stride, state_dtype, out, eps, scale, mode, workspace,
                          workspace_bytes, stream);
}

int gdn_prefill_chunked(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                        int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                        int64_t v_stride, int io_dtype, const float *g, const float *beta,
                        const int32_t *cu_seqlens, const int32_t *slot_in,
                        const int32_t *slot_out, int num_rows, void *ssm_pool,
                        int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                        float scale, int mode, void *workspace, size_t workspace_bytes,
                        void *stream)
{
    return prefill_common(false, N, T, H_qk, H_v, d_k, d_v, q, q_stride, k, k_stride, v, v_stride,
                          io_dtype, g, beta, cu_seqlens, slot_in, slot_out, num_rows, ssm_pool,
                          ssm_slot_stride, state_dtype, out, eps, scale, mode, workspace,
                          workspace_bytes, stream);
}

int kda_prefill_conv(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *x,
                     int io_dtype, const float *conv_w, const float *conv_b, void *conv_pool,
                     int64_t conv_slot_stride, int conv_dtype, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const int32_t *slot_in,
                     const int32_t *slot_out, int num_rows, void *ssm_pool,
                     int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                     float scale, int mode, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    const ConvIn cv{x, conv_w, conv_b, conv_pool, conv_slot_stride, conv_dtype};
    return prefill_common(true, N, T, H_qk, H_v, d_k, d_v, nullptr, 0, nullptr, 0, nullptr, 0,
                          io_dtype, g, beta, cu_seqlens, slot_in, slot_out, num_rows, ssm_pool,
                          ssm_slot_stride, state_dtype, out, eps, scale, mode, workspace,
                          workspace_bytes, stream, &cv);
}

int gdn_prefill_conv(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *x,
                     int io_dtype, const float *conv_w, const float *conv_b, void *conv_pool,
                     int64_t conv_slot_stride, int conv_dtype, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const int32_t *slot_in,
                     const int32_t *slot_out, int num_rows, void *ssm_pool,
                     int64_t ssm_slot_stride, int state_dtype, void *out, float eps,
                     float scale, int mode, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    const ConvIn cv{x, conv_w, conv_b, conv_pool, conv_slot_stride, conv_dtype};
    return prefill_common(false, N, T, H_qk, H_v, d_k, d_v, nullptr, 0, nullptr, 0, nullptr, 0,
                          io_dtype, g, beta, cu_seqlens, slot_in, slot_out, num_rows, ssm_pool,
                          ssm_slot_stride, state_dtype, out, eps, scale, mode, workspace,
                          workspace_bytes, stream, &cv);
}

static size_t prefill_ws(int N, int T, int H_qk, int H_v, int d_k, int d_v, int mode)
{
    if (N < 0 || T < 0 || H_qk <= 0 || H_v <= 0 || H_v % H_qk || d_k != d_v) return 0;
    if (mode != LA_PREFILL_FP32 && mode != LA_PREFILL_BF16X3) return 0;
    return la::prefill_ws_bytes(N, T, H_qk, H_v, d_k, mode);
}

int kda_prefill_chunked_noalloc(int N, int T, int H_qk, int H_v, int d_k, int d_v, const void *q,
                                int64_t q_stride, const void *k, int64_t k_stride, const void *v,
                                int64_t v_stride, int io_dtype, const float *g,
                                const float *beta, const int32_t *cu_seqlens,
                                const int32_t *slot_in, const int32_t *slot_out, int num_rows,
                                void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
                                void *out, float eps, float scale, int mode, void *stream)
{
    const char *fn = "kda_prefill_chunked_noalloc";
    const size_t need = prefill_ws(N, T, H_qk, H_v, d_k, d_v, mode);
    if (need > kScratchBytes)
        return fail(LA_ERR_WORKSPACE,
                    "%s: %d tokens x %d value heads need %zu bytes of scratch; this call holds "
                    "%zu (128 MiB) per GPU -- use kda_prefill_chunked with a workspace",
                    fn, T, H_v, need, kScratchBytes);
    void *ws = nullptr;
    if (need) {
        ws = scratch_address(fn);
        if (!ws) return LA_ERR_HIP;
    }
    return prefill_common(true, N, T, H_qk, H_v, d_k, d_v, q, q_stride, k, k_stride, v, v_stride,
                          io_dtype, g, beta, cu_seqlens, slot_in, slot_out, num_rows, ssm_pool,
                          ssm_slot_stride, state_dtype, out, eps, scale, mode, ws,
                          need ? kScratchBytes : 0, stream, nullptr, /*may_check=*/false);
}

size_t kda_prefill_workspace_bytes(int N, int T, int H_qk, int H_v, int d_k, int d_v, int mode)
{
    return prefill_ws(N, T, H_qk, H_v, d_k, d_v, mode);
}

size_t gdn_prefill_workspace_bytes(int N, int T, int H_qk, int H_v, int d_k, int d_v, int mode)
{
    return prefill_ws(N, T, H_qk, H_v, d_k, d_v, mode);
}

int la_ring_bytes(int layers, int slots, int H_v, int L, int d_k, int d_v, int io_dtype, int kda,
                  int64_t *d_bytes, int64_t *k_bytes, int64_t *g_bytes, int64_t *beta_bytes)
{
    if (layers < 0 || slots < 0 || H_v < 0 || L < 0 || d_k < 0 || d_v < 0)
        return fail(LA_ERR_ARG, "la_ring_bytes: negative size");
    if (!valid_dtype(io_dtype))
        return fail(LA_ERR_ARG, "la_ring_bytes: io_dtype must be LA_F32 or LA_BF16");
    const int64_t steps = (int64_t)layers * (slots + 1) * H_v * L;  // records per buffer
    if (d_bytes) *d_bytes = steps * d_v * dsize(io_dtype);
    if (k_bytes) *k_bytes = steps * d_k * dsize(io_dtype);
    if (g_bytes) *g_bytes = steps * (kda ? d_k : 1) * (int64_t)sizeof(float);
    if (beta_bytes) *beta_bytes = steps * (int64_t)sizeof(float);
    return ok();
}


int kda_verify(int B, int D, const int32_t *n_tok, int H_qk, int H_v, int d_k, int d_v,
               const void *x, int io_dtype, const float *conv_w, const float *conv_b,
               const void *conv_pool, int64_t conv_slot_stride, int conv_dtype, const float *g,
               const float *beta, const int32_t *slots, int num_rows, const void *ssm_pool,
               int64_t ssm_slot_stride, int state_dtype, void *out, void *conv_windows,
               const la_ring *ring, const int32_t *ring_base, float eps, float scale,
               void *stream)
{
    return verify_common(true, B, D, n_tok, H_qk, H_v, d_k, d_v, x, io_dtype, conv_w, conv_b,
                         conv_pool, conv_slot_stride, conv_dtype, g, beta, slots, num_rows,
                         ssm_pool, ssm_slot_stride, state_dtype, out, conv_windows, ring,
                         ring_base, eps, scale, stream);
}

int gdn_verify(int B, int D, const int32_t *n_tok, int H_qk, int H_v, int d_k, int d_v,
               const void *x, int io_dtype, const float *conv_w, const float *conv_b,
               const void *conv_pool, int64_t conv_slot_stride, int conv_dtype, const float *g,
               const float *beta, const int32_t *slots, int num_rows, const void *ssm_pool,
               int64_t ssm_slot_stride, int state_dtype, void *out, void *conv_windows,
               const la_ring *ring, const int32_t *ring_base, float eps, float scale,
               void *stream)
{
    return verify_common(false, B, D, n_tok, H_qk, H_v, d_k, d_v, x, io_dtype, conv_w, conv_b,
                         conv_pool, conv_slot_stride, conv_dtype, g, beta, slots, num_rows,
                         ssm_pool, ssm_slot_stride, state_dtype, out, conv_windows, ring,
                         ring_base, eps, scale, stream);
}

int kda_commit(int B, const int32_t *accepted, int H_v, int d_k, int d_v, const int32_t *slots,
               int num_rows, void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
               int io_dtype, const la_ring *ring, const int32_t *ring_base, float eps,
               void *stream)
{
    return commit_common(true, B, accepted, H_v, d_k, d_v, slots, num_rows, ssm_pool,
                         ssm_slot_stride, state_dtype, io_dtype, ring, ring_base, eps, stream);
}

int gdn_commit(int B, const int32_t *accepted, int H_v, int d_k, int d_v, const int32_t *slots,
               int num_rows, void *ssm_pool, int64_t ssm_slot_stride, int state_dtype,
               int io_dtype, const la_ring *ring, const int32_t *ring_base, float eps,
               void *stream)
{
    return commit_common(false, B, accepted, H_v, d_k, d_v, slots, num_rows, ssm_pool,
                         ssm_slot_stride, state_dtype, io_dtype, ring, ring_base, eps, stream);
}

int conv_window_scatter(int B, int D, int C, const uint8_t *mask, const int32_t *slots,
                        const int32_t *step, const void *windows, void *conv_pool,
                        int64_t conv_slot_stride, int conv_dtype, int num_rows, void *stream)
{
    const char *fn = "conv_window_scatter";
    if (B < 0 || D <= 0 || C <= 0 || num_rows <= 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be positive (B >= 0)", fn);
    if (!valid_dtype(conv_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    if ((3LL * C * dsize(conv_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: a window (3 C elements) must be a multiple of 16 bytes", fn);
    if (B == 0) return ok();
    if (!slots || !step || !windows || !conv_pool)
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {slots, step, windows, conv_pool};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    if (conv_slot_stride < 3LL * C || (conv_slot_stride * dsize(conv_dtype)) % 16)
        return fail(LA_ERR_ARG, "%s: conv_slot_stride %lld too small or misaligned", fn,
                    (long long)conv_slot_stride);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(slots, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "slots")) return rc;
    }
    la::ScatterArgs a{};
    a.B = B; a.D = D; a.C = C; a.mask = mask; a.slots = slots; a.step = step; a.windows = windows;
    a.conv_pool = conv_pool; a.conv_stride = conv_slot_stride; a.conv_dtype = conv_dtype;
    a.num_rows = num_rows;
    return hip_status(la::launch_conv_scatter(a, st), fn);
}

int state_track_copy(int B, const uint8_t *mask, const int32_t *src, const int32_t *dst,
                     void *conv_pool, int64_t conv_slot_stride, int64_t conv_row_elems,
                     int conv_dtype, void *ssm_pool, int64_t ssm_slot_stride,
                     int64_t ssm_row_elems, int state_dtype, int num_rows, void *stream)
{
    const char *fn = "state_track_copy";
    if (B < 0 || num_rows <= 0 || conv_row_elems < 0 || ssm_row_elems < 0)
        return fail(LA_ERR_ARG, "%s: dimensions must be non-negative", fn);
    if (!valid_dtype(conv_dtype) || !valid_dtype(state_dtype))
        return fail(LA_ERR_UNSUPPORTED, "%s: dtype codes must be LA_F32 or LA_BF16", fn);
    const int64_t crow = conv_row_elems * dsize(conv_dtype), srow = ssm_row_elems * dsize(state_dtype);
    if (crow % 16 || srow % 16)
        return fail(LA_ERR_ARG, "%s: rows must be multiples of 16 bytes", fn);
    if (B == 0) return ok();
    if (!src || !dst || (crow && !conv_pool) || (srow && !ssm_pool))
        return fail(LA_ERR_ARG, "%s: null pointer argument", fn);
    const void *ptrs[] = {src, dst, conv_pool, ssm_pool};  // mask: bytes, any alignment
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return fail(LA_ERR_ARG, "%s: pointers must be 16-byte aligned", fn);
    if ((crow && (conv_slot_stride < conv_row_elems || (conv_slot_stride * dsize(conv_dtype)) % 16)) ||
        (srow && (ssm_slot_stride < ssm_row_elems || (ssm_slot_stride * dsize(state_dtype)) % 16)))
        return fail(LA_ERR_ARG, "%s: slot strides must cover a row and be multiples of 16 bytes",
                    fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (checked_mode()) {
        std::vector<int32_t> hs;
        if (int rc = fetch_i32(dst, B, hs, st)) return rc;
        if (int rc = check_slots(hs, num_rows, false, "dst")) return rc;
    }
    la::TrackArgs a{};
    a.B = B; a.mask = mask; a.src = src; a.dst = dst;
    a.conv_pool = static_cast<char *>(conv_pool); a.ssm_pool = static_cast<char *>(ssm_pool);
    a.conv_stride_b = conv_slot_stride * dsize(conv_dtype); a.conv_row_b = crow;
    a.ssm_stride_b = ssm_slot_stride * dsize(state_dtype); a.ssm_row_b = srow;
    a.num_rows = num_rows;
    return hip_status(la::launch_track_copy(a, st), fn);
}

int kda_ring_fold(int B, const int32_t *m, int H_v, int d_k, int d_v, const int32_t *slots,
                  const int32_t *dst_slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                  const void *q, void *out, float eps, float scale, void *stream)
{
    return fold_common(true, B, m, H_v, d_k, d_v, slots, dst_slots, num_rows, ssm_pool,
                       ssm_slot_stride, state_dtype, io_dtype, ring, ring_base, q, out, eps, scale,
                       stream);
}

int gdn_ring_fold(int B, const int32_t *m, int H_v, int d_k, int d_v, const int32_t *slots,
                  const int32_t *dst_slots, int num_rows, void *ssm_pool, int64_t ssm_slot_stride,
                  int state_dtype, int io_dtype, const la_ring *ring, const int32_t *ring_base,
                  const void *q, void *out, float eps, float scale, void *stream)
{
    return fold_common(false, B, m, H_v, d_k, d_v, slots, dst_slots, num_rows, ssm_pool,
                       ssm_slot_stride, state_dtype, io_dtype, ring, ring_base, q, out, eps, scale,
                       stream);
}
}  // extern "C"
