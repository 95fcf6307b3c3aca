"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant, a library
routine (numpy/scipy/torch) or a brute-force formulation that is written
differently from the oracle (explicit products of the per-token transition
matrices), so that a dropped term, a wrong sign or index, a transposed
operand or a wrong tap order fails at least one of them.

Sources: the gated delta rule as the decode kernel's steps ("SGLang之KV
Cache内存池机制", section 8.5) and as the ReplaySSM exact-commit replay and
the fast-rebuild unrolled sum (xxmr.cn/news/181459, ReplaySSM passages); the
short conv ("Conv state" passage of the same page; hotelren.com/news/5417338
section 2.1).
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from linear_attention_recurrent_amd import synth

EPS = 1e-6


def silu_lib(y):
    return y * scipy.special.expit(y)


def l2n(x, eps=EPS):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------- codec ----

def test_round_fp32_matches_numpy_cast():
    x = synth.normal(1, 0, (4096,)) * np.exp(synth.normal(1, 1, (4096,)) * 20)
    assert np.array_equal(oracle.round_to(x, "fp32"), x.astype(np.float32).astype(np.float64))


def test_round_bf16_matches_torch_on_fp32_values():
    # For values already exact in fp32 there is no double rounding, so the
    # direct fp64->bf16 rounding must equal torch's fp32->bf16 conversion.
    raw = synth.raw_u64(2, 0, 20000)
    bits = (raw >> np.uint64(32)).astype(np.uint32)
    x32 = bits.view(np.float32)
    x32 = x32[np.isfinite(x32) & (np.abs(x32) < 3e38)]
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_round_bf16_ties_and_specials():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                    # tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,      # tie -> even (1 + 2^-6)
        one + ulp / 2 + 2.0 ** -30: one + ulp, # just above the tie
        -(one + ulp / 2): -one,
        0.0: 0.0,
        2.0 ** -133: 2.0 ** -133,              # smallest bf16 subnormal
        2.0 ** -134: 0.0,                      # tie at half the smallest subnormal -> 0 (even)
        3e38 * 1.2: np.inf,
    }
    for x, want in cases.items():
        assert oracle.round_to(np.array([x]), "bf16")[0] == want, x


# ----------------------------------------------------------------- conv ----

def _conv_direct(x, w, hist):
    """Library-based direct 4-tap causal cross-correlation per channel:
    np.convolve with the reversed taps over [history | x]."""
    T, C = x.shape
    y = np.empty((T, C))
    for c in range(C):
        xp = np.concatenate([hist[:, c], x[:, c]])
        y[:, c] = np.convolve(xp, w[c, ::-1], mode="valid")
    return y


def test_conv_impulse_reveals_tap_order():
    C = 5
    w = synth.normal(3, 0, (C, 4))
    x = np.zeros((6, C))
    x[0, :] = 1.0
    y, _ = oracle.shortconv_prefill(x, [0, 6], [-1], [1], w, None, np.zeros((2, 3, C)),
                                    io_dtype="fp64")
    # Impulse at token 0: token t sees it at window position 3 - t.
    for t in range(4):
        np.testing.assert_allclose(y[t], silu_lib(w[:, 3 - t]), rtol=1e-14, atol=0)
    np.testing.assert_array_equal(y[4:], 0.0)


def test_conv_prefill_matches_np_convolve_and_history_roll():
    C, T = 7, 11
    x = synth.normal(4, 0, (T, C))
    w = synth.normal(4, 1, (C, 4)) * 0.5
    b = synth.normal(4, 2, (C,))
    pool = synth.normal(4, 3, (4, 3, C))
    y, newpool = oracle.shortconv_prefill(x, [0, T], [2], [3], w, b, pool, io_dtype="fp64",
                                          conv_dtype="fp64")
    ref = silu_lib(_conv_direct(x, w, pool[2]) + b)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)
    # slot_out holds the last three inputs exactly; other rows untouched.
    np.testing.assert_array_equal(newpool[3], x[-3:])
    np.testing.assert_array_equal(newpool[:3], pool[:3])


def test_conv_short_sequence_shifts_in_old_history():
    C = 3
    pool = synth.normal(5, 0, (3, 3, C))
    x = synth.normal(5, 1, (2, C))
    w = synth.normal(5, 2, (C, 4))
    _, newpool = oracle.shortconv_prefill(x, [0, 2], [1], [2], w, None, pool, conv_dtype="fp64")
    np.testing.assert_array_equal(newpool[2], np.stack([pool[1][2], x[0], x[1]]))


def test_conv_dtype_only_rounds_the_handoff():
    """Inside one call the window holds the sequence's own inputs: with no
    prior history the conv-state dtype cannot change the outputs, and only the
    three inputs handed to slot_out are rounded to it.  Splitting a sequence
    over two calls through an fp64 history reproduces the single call."""
    C, T = 6, 9
    x = synth.normal(7, 0, (T, C)) * 1.37  # not representable in bf16
    w = synth.normal(7, 1, (C, 4))
    pool = np.zeros((3, 3, C))
    y64, p64 = oracle.shortconv_prefill(x, [0, T], [-1], [1], w, None, pool, conv_dtype="fp64",
                                        io_dtype="fp64")
    ybf, pbf = oracle.shortconv_prefill(x, [0, T], [-1], [1], w, None, pool, conv_dtype="bf16",
                                        io_dtype="fp64")
    np.testing.assert_array_equal(ybf, y64)
    np.testing.assert_array_equal(pbf[1], oracle.round_to(x[-3:], "bf16"))
    assert not np.array_equal(pbf[1], p64[1])
    for cut in (1, 2, 5):
        ya, pa = oracle.shortconv_prefill(x[:cut], [0, cut], [-1], [1], w, None, pool,
                                          conv_dtype="fp64", io_dtype="fp64")
        yb, pb = oracle.shortconv_prefill(x[cut:], [0, T - cut], [1], [2], w, None, pa,
                                          conv_dtype="fp64", io_dtype="fp64")
        np.testing.assert_array_equal(np.concatenate([ya, yb]), y64)
        np.testing.assert_array_equal(pb[2], p64[1])


def test_conv_decode_step_matches_direct_sum():
    B, C, P = 4, 9, 6
    x = synth.normal(6, 0, (B, C))
    w = synth.normal(6, 1, (C, 4))
    pool = synth.normal(6, 2, (P + 1, 3, C))
    slots = np.array([3, 1, 6, 2], dtype=np.int32)
    y, newpool = oracle.shortconv_step(x, w, None, pool, slots, conv_dtype="fp64")
    for bi, s in enumerate(slots):
        ref = silu_lib(_conv_direct(x[bi:bi + 1], w, pool[s])[0])
        np.testing.assert_allclose(y[bi], ref, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(newpool[s], np.concatenate([pool[s][1:], x[bi:bi + 1]]))
    untouched = [r for r in range(P + 1) if r not in set(slots.tolist())]
    np.testing.assert_array_equal(newpool[untouched], pool[untouched])


# ------------------------------------------------------ recurrence pins ----

def _rand_step(seed, B, H, d, kda=True, Hv=None):
    Hv = Hv or H
    q = synth.normal(seed, 0, (B, H, d))
    k = synth.normal(seed, 1, (B, H, d))
    v = synth.normal(seed, 2, (B, Hv, d))
    g = synth.log_decay(seed, 3, (B, Hv, d) if kda else (B, Hv)).astype(np.float64)
    beta = synth.beta_gate(seed, 4, (B, Hv)).astype(np.float64)
    return q, k, v, g, beta


def test_alpha_one_beta_zero_leaves_state_unchanged():
    B, H, d, P = 3, 2, 16, 4
    q, k, v, g, beta = _rand_step(10, B, H, d)
    pool = synth.normal(10, 5, (P + 1, H, d, d))
    slots = [2, 4, 1]
    for kda in (True, False):
        gg = np.zeros_like(g) if kda else np.zeros((B, H))
        out, newpool = oracle.recurrent_step(q, k, v, gg, np.zeros_like(beta), slots, pool,
                                             kda=kda, state_dtype="fp64", io_dtype="fp64")
        np.testing.assert_array_equal(newpool, pool)
        for bi, s in enumerate(slots):
            o_ref = np.einsum("hij,hj->hi", pool[s], l2n(q[bi]))
            np.testing.assert_allclose(out[bi], o_ref, rtol=1e-12, atol=1e-13)


def test_first_step_from_zero_state_closed_form_and_l2norm():
    # S_1 = beta v k^T, o_1 = beta (k.q) v, and |k_hat|^2 = s / (s + eps).
    B, H, d = 2, 3, 16
    q, k, v, g, beta = _rand_step(11, B, H, d)
    k[0, 0] *= 1e-3  # small key: eps visibly matters
    pool = np.zeros((B + 1, H, d, d))
    out, newpool = oracle.recurrent_step(q, k, v, g, beta, [1, 2], pool,
                                         state_dtype="fp64", io_dtype="fp64")
    for bi in range(B):
        S = newpool[bi + 1]
        s = np.sum(k[bi] ** 2, axis=-1)
        khat = k[bi] / np.sqrt(s + EPS)[:, None]
        qhat = q[bi] / np.sqrt(np.sum(q[bi] ** 2, axis=-1) + EPS)[:, None]
        S_ref = beta[bi][:, None, None] * v[bi][:, :, None] * khat[:, None, :]
        np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-15)
        o_ref = beta[bi][:, None] * np.sum(khat * qhat, -1)[:, None] * v[bi]
        np.testing.assert_allclose(out[bi], o_ref, rtol=1e-12, atol=1e-15)
        # recover k_hat from a row of S and check its norm closed form
        kr = S[:, 0, :] / (beta[bi][:, None] * v[bi][:, 0:1])
        np.testing.assert_allclose(np.sum(kr ** 2, -1), s / (s + EPS), rtol=1e-10)


def test_beta_one_writes_v_along_k():
    # beta=1: S_t k_hat - v = (S' k_hat - v) * eps / (s + eps)  (closed form)
    B, H, d, P = 2, 2, 32, 3
    q, k, v, g, _ = _rand_step(12, B, H, d)
    pool = synth.normal(12, 5, (P + 1, H, d, d))
    slots = [3, 1]
    _, newpool = oracle.recurrent_step(q, k, v, g, np.ones((B, H)), slots, pool,
                                       state_dtype="fp64", io_dtype="fp64")
    for bi, s in enumerate(slots):
        ss = np.sum(k[bi] ** 2, -1)
        khat = k[bi] / np.sqrt(ss + EPS)[:, None]
        Sprime = pool[s] * np.exp(g[bi])[:, None, :]
        resid_before = np.einsum("hij,hj->hi", Sprime, khat) - v[bi]
        resid_after = np.einsum("hij,hj->hi", newpool[s], khat) - v[bi]
        np.testing.assert_allclose(resid_after, resid_before * (EPS / (ss + EPS))[:, None],
                                   rtol=1e-6, atol=1e-12)
        assert np.max(np.abs(resid_after)) < 1e-6


@pytest.mark.parametrize("kda", [True, False])
def test_decay_only_steps_compose_multiplicatively(kda):
    B, H, d, n = 1, 2, 16, 20
    pool0 = synth.normal(13, 5, (2, H, d, d))
    pool = pool0.copy()
    gsum = 0.0
    for t in range(n):
        q, k, v, g, beta = _rand_step(100 + t, B, H, d, kda)
        _, pool = oracle.recurrent_step(q, k, v, g, np.zeros_like(beta), [1], pool, kda=kda,
                                        state_dtype="fp64", io_dtype="fp64")
        gsum = gsum + g[0]
    decay = np.exp(gsum)[:, None, :] if kda else np.exp(gsum)[:, None, None]
    np.testing.assert_allclose(pool[1], pool0[1] * decay, rtol=4 * n * 2.0 ** -52, atol=0)


def _transition_product_reference(S0, qs, ks, vs, alphas, betas, scale=1.0):
    """Brute force: S_T = S_0 M_1...M_T + sum_t beta_t v_t k_t^T M_{t+1}...M_T
    with M_t = Diag(alpha_t)(I - beta_t k_t k_t^T), for q/k already normalised.
    Returns all outputs o_t = scale S_t q_t and S_T."""
    T, d = ks.shape
    outs = []
    for t in range(T):
        Ms = [np.diag(alphas[j]) @ (np.eye(d) - betas[j] * np.outer(ks[j], ks[j]))
              for j in range(t + 1)]
        prod = np.eye(d)
        for M in Ms:
            prod = prod @ M
        S = S0 @ prod
        for j in range(t + 1):
            tail = np.eye(d)
            for M in Ms[j + 1:]:
                tail = tail @ M
            S = S + betas[j] * np.outer(vs[j], ks[j]) @ tail
        outs.append(scale * S @ qs[t])
    return np.array(outs), S


@pytest.mark.parametrize("kda", [True, False])
def test_brute_force_transition_products_tiny(kda):
    # d=16, T=64 sequential tokens (the tiny GDN-style layer), one head.
    T, d = 64, 16
    q = synth.normal(20, 0, (T, 1, d))
    k = synth.normal(20, 1, (T, 1, d))
    v = synth.normal(20, 2, (T, 1, d))
    g = synth.log_decay(20, 3, (T, 1, d) if kda else (T, 1)).astype(np.float64)
    beta = synth.beta_gate(20, 4, (T, 1)).astype(np.float64)
    S0 = synth.normal(20, 5, (d, d))
    pool = np.zeros((2, 1, d, d))
    pool[1, 0] = S0
    out, newpool = oracle.prefill(q, k, v, g, beta, [0, T], [1], [1], pool, kda=kda,
                                  state_dtype="fp64", io_dtype="fp64", scale=0.5)
    alphas = np.exp(g[:, 0] if kda else np.repeat(g[:, 0:1], d, axis=1))
    o_ref, S_ref = _transition_product_reference(S0, l2n(q[:, 0]), l2n(k[:, 0]), v[:, 0],
                                                 alphas, beta[:, 0], scale=0.5)
    np.testing.assert_allclose(newpool[1, 0], S_ref, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(out[:, 0], o_ref, rtol=1e-10, atol=1e-11)


def test_tiny_gdn_layer_full_pipeline_brute_force():
    """The whole decode definition on the tiny GDN layer (B=1, H=2, d=16,
    T=64 decode steps, conv weights 0.5*randn, zero initial state): numpy
    conv + scipy SiLU + explicit transition products vs 64 oracle steps."""
    H, d, T = 2, 16, 64
    sh = synth.DecodeShape(B=1, Hqk=H, Hv=H, dk=d, dv=d, P=1, kda=False,
                           io="fp32", state="fp32", conv="fp32")
    C = sh.C
    w = 0.5 * synth.normal(1000, synth.S_W, (C, 4))
    xs = synth.normal(1000, synth.S_X, (T, C))
    g = synth.log_decay(1000, synth.S_G, (T, H)).astype(np.float64)
    beta = synth.beta_gate(1000, synth.S_BETA, (T, H)).astype(np.float64)
    conv_pool = np.zeros((2, 3, C))
    ssm_pool = np.zeros((2, H, d, d))
    outs = []
    for t in range(T):
        o, conv_pool, ssm_pool = oracle.decode(xs[t:t + 1], w, None, conv_pool, g[t:t + 1],
                                               beta[t:t + 1], [1], ssm_pool, Hqk=H, Hv=H,
                                               dk=d, dv=d, kda=False, state_dtype="fp64",
                                               io_dtype="fp64", conv_dtype="fp64")
        outs.append(o[0])
    outs = np.array(outs)
    y = silu_lib(_conv_direct(xs, w, np.zeros((3, C))))
    for h in range(H):
        qh = l2n(y[:, h * d:(h + 1) * d])
        kh = l2n(y[:, H * d + h * d:H * d + (h + 1) * d])
        vh = y[:, 2 * H * d + h * d:2 * H * d + (h + 1) * d]
        o_ref, S_ref = _transition_product_reference(
            np.zeros((d, d)), qh, kh, vh, np.exp(np.repeat(g[:, h:h + 1], d, 1)), beta[:, h])
        np.testing.assert_allclose(ssm_pool[1, h], S_ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(outs[:, h], o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(conv_pool[1], xs[-3:])


def test_unrolled_sum_of_the_fast_rebuild():
    """S_m = S_0 Diag(prod alpha) + sum_j d_j (k_j . prod_{i>j} alpha_i)^T with
    d_j = beta_j (v_j - S_{j-1} Diag(alpha_j) k_j) read off the oracle's own
    per-step states (xxmr.cn ReplaySSM fast-rebuild passage)."""
    m, d = 12, 16
    S_prev = synth.normal(30, 5, (d, d))
    S0 = S_prev.copy()
    ds, ks, alphas = [], [], []
    pool = np.zeros((2, 1, d, d))
    pool[1, 0] = S0
    for j in range(m):
        q, k, v, g, beta = _rand_step(300 + j, 1, 1, d)
        _, pool = oracle.recurrent_step(q, k, v, g, beta, [1], pool,
                                        state_dtype="fp64", io_dtype="fp64")
        khat = l2n(k[0, 0])
        alpha = np.exp(g[0, 0])
        S_new = pool[1, 0]
        # d_j from the definition, using the oracle's previous state
        d_j = beta[0, 0] * (v[0, 0] - (S_prev * alpha) @ khat)
        np.testing.assert_allclose(S_new, S_prev * alpha + np.outer(d_j, khat), rtol=1e-12,
                                   atol=1e-13)
        ds.append(d_j); ks.append(khat); alphas.append(alpha)
        S_prev = S_new
    S_m = S0 * np.prod(alphas, axis=0)
    for j in range(m):
        tail = np.prod(alphas[j + 1:], axis=0) if j + 1 < m else np.ones(d)
        S_m = S_m + np.outer(ds[j], ks[j] * tail)
    np.testing.assert_allclose(pool[1, 0], S_m, rtol=1e-11, atol=1e-12)


def test_gdn_equals_kda_with_broadcast_gate():
    B, Hqk, Hv, d, P = 3, 2, 4, 16, 5
    q, k, _, _, _ = _rand_step(40, B, Hqk, d)
    v = synth.normal(40, 2, (B, Hv, d))
    g = synth.log_decay(40, 3, (B, Hv)).astype(np.float64)
    beta = synth.beta_gate(40, 4, (B, Hv)).astype(np.float64)
    pool = synth.normal(40, 5, (P + 1, Hv, d, d))
    slots = [5, 2, 3]
    o1, p1 = oracle.recurrent_step(q, k, v, g, beta, slots, pool, kda=False,
                                   state_dtype="fp64", io_dtype="fp64")
    o2, p2 = oracle.recurrent_step(q, k, v, np.repeat(g[:, :, None], d, 2), beta, slots, pool,
                                   kda=True, state_dtype="fp64", io_dtype="fp64")
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(p1, p2, rtol=1e-13, atol=1e-14)


def test_gqa_head_map_consecutive_grouping():
    # value head h reads q/k head h // (Hv/Hqk): permuting k heads moves the
    # affected value heads accordingly.
    B, Hqk, Hv, d = 1, 2, 4, 8
    q, k, _, _, _ = _rand_step(41, B, Hqk, d)
    v = synth.normal(41, 2, (B, Hv, d))
    g = synth.log_decay(41, 3, (B, Hv, d)).astype(np.float64)
    beta = synth.beta_gate(41, 4, (B, Hv)).astype(np.float64)
    pool = synth.normal(41, 5, (2, Hv, d, d))
    o, p = oracle.recurrent_step(q, k, v, g, beta, [1], pool, state_dtype="fp64",
                                 io_dtype="fp64")
    for h in range(Hv):
        oh, ph = oracle.recurrent_step(q[:, h // 2:h // 2 + 1], k[:, h // 2:h // 2 + 1],
                                       v[:, h:h + 1], g[:, h:h + 1], beta[:, h:h + 1], [1],
                                       pool[:, h:h + 1], state_dtype="fp64", io_dtype="fp64")
        np.testing.assert_array_equal(o[:, h], oh[:, 0])
        np.testing.assert_array_equal(p[1, h], ph[1, 0])


def test_rows_evolve_independently_and_untouched_rows_stay():
    B, H, d, P = 2, 2, 16, 6
    q, k, v, g, beta = _rand_step(50, B, H, d)
    pool = synth.normal(50, 5, (P + 1, H, d, d)).astype(np.float32).astype(np.float64)
    slots = [4, 2]
    o1, p1 = oracle.recurrent_step(q, k, v, g, beta, slots, pool)
    v2 = v.copy()
    v2[1, 0, 7] += 1.0
    o2, p2 = oracle.recurrent_step(q, k, v2, g, beta, slots, pool)
    changed_rows = np.any(p1[2, 0] != p2[2, 0], axis=1)
    assert changed_rows.tolist() == [i == 7 for i in range(d)]
    assert np.array_equal(o1[1, 0] != o2[1, 0], np.arange(d) == 7)
    np.testing.assert_array_equal(p1[[0, 1, 3, 5, 6]], pool[[0, 1, 3, 5, 6]])
    # batch permutation with its slots gives identical pools and permuted outputs
    perm = [1, 0]
    o3, p3 = oracle.recurrent_step(q[perm], k[perm], v[perm], g[perm], beta[perm],
                                   [slots[i] for i in perm], pool)
    np.testing.assert_array_equal(p3, p1)
    np.testing.assert_array_equal(o3, o1[perm])


def test_bf16_state_is_rounded_every_token():
    B, H, d = 1, 1, 16
    q, k, v, g, beta = _rand_step(60, B, H, d)
    pool = oracle.round_to(synth.normal(60, 5, (2, H, d, d)), "bf16")
    _, p32 = oracle.recurrent_step(q, k, v, g, beta, [1], pool, state_dtype="fp64")
    _, p16 = oracle.recurrent_step(q, k, v, g, beta, [1], pool, state_dtype="bf16")
    np.testing.assert_array_equal(p16, oracle.round_to(p32, "bf16"))


# ---------------------------------------------------------------- prefill --

def test_prefill_equals_sequential_decode_steps():
    T, H, d = 9, 2, 16
    q = synth.normal(70, 0, (T, H, d))
    k = synth.normal(70, 1, (T, H, d))
    v = synth.normal(70, 2, (T, H, d))
    g = synth.log_decay(70, 3, (T, H, d)).astype(np.float64)
    beta = synth.beta_gate(70, 4, (T, H)).astype(np.float64)
    pool = np.zeros((3, H, d, d))
    pool[1] = synth.normal(70, 5, (H, d, d))
    out, newpool = oracle.prefill(q, k, v, g, beta, [0, T], [1], [2], pool,
                                  state_dtype="fp64", io_dtype="fp64")
    dpool = pool.copy()
    for t in range(T):
        o, dpool = oracle.recurrent_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                         beta[t:t + 1], [1], dpool, state_dtype="fp64",
                                         io_dtype="fp64")
        np.testing.assert_allclose(out[t], o[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(newpool[2], dpool[1], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(newpool[1], pool[1])   # slot_in untouched


def test_prefill_packing_and_split_invariance():
    H, d = 2, 16
    lens = [5, 1, 7]
    T = sum(lens)
    q = synth.normal(71, 0, (T, H, d))
    k = synth.normal(71, 1, (T, H, d))
    v = synth.normal(71, 2, (T, H, d))
    g = synth.log_decay(71, 3, (T, H, d)).astype(np.float64)
    beta = synth.beta_gate(71, 4, (T, H)).astype(np.float64)
    pool = np.zeros((5, H, d, d))
    cu = synth.cu_seqlens(lens)
    out, p = oracle.prefill(q, k, v, g, beta, cu, [-1, -1, -1], [1, 2, 3], pool)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        o1, p1 = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a], [-1],
                                [4], pool)
        np.testing.assert_array_equal(o1, out[a:b])
        np.testing.assert_array_equal(p1[4], p[n + 1])
    # split the 7-token sequence 3 + 4 through a pool slot (fp32 hand-off)
    a = cu[2]
    o_a, pa = oracle.prefill(q[a:a + 3], k[a:a + 3], v[a:a + 3], g[a:a + 3], beta[a:a + 3],
                             [0, 3], [-1], [4], pool)
    o_b, pb = oracle.prefill(q[a + 3:], k[a + 3:], v[a + 3:], g[a + 3:], beta[a + 3:],
                             [0, 4], [4], [4], pa)
    np.testing.assert_allclose(np.concatenate([o_a, o_b]), out[a:], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(pb[4], p[3], rtol=1e-6, atol=1e-7)
