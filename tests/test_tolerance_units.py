"""Why prefill outputs are compared per (sequence, head) and not per token.

Under strong decay a token's output is about (q_t . k_t) beta_t v_t: the
state it reads holds almost nothing but the token's own update.  When q_t
and k_t are nearly orthogonal that output is a cancellation, and its
relative error is the absolute error of the dot product over |q_t . k_t|.
No fixed-precision evaluation stays within a relative bound of such a
token: the plain token-by-token recurrence ("SGLang之KV Cache内存池机制"
section 8.5: decay, delta, rank-one update, read-out) run in fp32 arithmetic
misses 1e-4 per token on g = -30 inputs, while it meets 1e-4 per (sequence,
head) with the element-wise floor at that unit's rms.  So the per-token unit
measures the input's conditioning, not an implementation; the GPU parity
tests take the (sequence, head) unit for prefill outputs.
"""
import numpy as np
import torch

import oracle
from linear_attention_recurrent_amd import synth
from parity_util import ELEM_TOL_SPLIT, TOL, elem_err, rel_err_units


def fp32_recurrence(q, k, v, g, beta, cu, S0):
    """The token-by-token recurrence in fp32 arithmetic (KDA gates)."""
    f = np.float32
    T, H, D = v.shape
    out = np.zeros((T, H, D), f)
    for n in range(len(cu) - 1):
        S = S0[n].astype(f).copy()
        for t in range(cu[n], cu[n + 1]):
            for h in range(H):
                qq, kk = q[t, h].astype(f), k[t, h].astype(f)
                qq = qq / np.sqrt((qq * qq).sum(dtype=f) + f(1e-6))
                kk = kk / np.sqrt((kk * kk).sum(dtype=f) + f(1e-6))
                Sp = S[h] * np.exp(g[t, h].astype(f))[None, :]
                d = f(beta[t, h]) * (v[t, h].astype(f) - Sp @ kk)
                S[h] = Sp + np.outer(d, kk)
                out[t, h] = S[h] @ qq
    return out


def seq_units(x, cu):
    """[T, H, d] -> list of [H, tokens, d] blocks, one per sequence."""
    return [np.swapaxes(x[cu[n]:cu[n + 1]], 0, 1) for n in range(len(cu) - 1)]


def test_fp32_recurrence_misses_the_per_token_bar_under_strong_decay():
    lens = [150, 40, 70]
    H, D = 2, 128
    sh = synth.PrefillShape(seqlens=tuple(lens), Hqk=H, Hv=H, dk=D, dv=D, io="fp32",
                            state="fp32")
    inp = synth.prefill_inputs(sh, 3010, "cpu")
    f = lambda name: inp[name].numpy().astype(np.float64)  # noqa: E731
    g = f("g")
    g[:lens[0]] = -30.0
    cu = synth.cu_seqlens(lens)
    S0 = synth.normal(3010, synth.S_SSM, (3, H, D, D)).astype(np.float32).astype(np.float64)
    pool = np.concatenate([np.zeros((1, H, D, D)), S0])
    si = np.array([1, 2, 3], np.int32)
    so = si
    o_ref, _ = oracle.prefill(f("q"), f("k"), f("v"), g, f("beta"), cu, si, so, pool,
                              kda=True, state_dtype="fp32", io_dtype="fp64")
    o32 = fp32_recurrence(f("q"), f("k"), f("v"), g, f("beta"), cu, S0)
    per_token = rel_err_units(o32, o_ref, 2)
    per_seq = max(rel_err_units(a, b, 1) for a, b in zip(seq_units(o32, cu), seq_units(o_ref, cu)))
    per_seq_el = max(elem_err(a, b, 1)[0]
                     for a, b in zip(seq_units(o32, cu), seq_units(o_ref, cu)))
    print(f"fp32 recurrence: per token {per_token:.2e}, per (sequence, head) {per_seq:.2e}, "
          f"element {per_seq_el:.2e}")
    assert per_token > 1e-4
    assert per_seq < 1e-5 and per_seq_el < 2e-5


# --- the element bar of the bf16x3 mode -------------------------------------

def _bf16(x):
    """Round fp32 values to bf16, nearest even (kept as fp32)."""
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def _mm(a, b, split):
    """a @ b exactly, or as the bf16x3 mode forms it: both fp32 operands split
    into bf16 hi + lo, the products lo.hi + hi.lo + hi.hi, an fp32 result."""
    if not split:
        return a @ b
    a, b = a.astype(np.float32), b.astype(np.float32)
    ah, bh = _bf16(a), _bf16(b)
    al, bl = _bf16(a - ah), _bf16(b - bh)
    f = lambda x: x.astype(np.float64)  # noqa: E731
    return (f(al) @ f(bh) + f(ah) @ f(bl) + f(ah) @ f(bh)).astype(np.float32).astype(np.float64)


def _chunked(q, k, v, g, beta, S0, split, CB=64):
    """One KDA sequence by blocks of CB tokens in the block form of the
    ReplaySSM fast-rebuild passage (xxmr.cn/news/181459): with G the running
    log decay inside the block, A_tj = beta_t sum_c k_t k_j e^(G_t - G_j)
    (j < t), T = (I + A)^-1, U = T (beta V), W = T (beta K e^G), D = U - W S^T,
    O = (Q e^G) S^T + P D with P_tj = sum_c q_t k_j e^(G_t - G_j) (j <= t),
    and S <- S e^(G_last) + D^T (K e^(G_last - G)).  The three contractions
    with the state (D, O and the update) take the split products when split."""
    T, D = q.shape
    nrm = lambda x: x / np.sqrt((x * x).sum(1, keepdims=True) + 1e-6)  # noqa: E731
    q, k = nrm(q), nrm(k)
    S, out = S0.copy(), np.zeros((T, D))
    for b0 in range(0, T, CB):
        s = slice(b0, min(T, b0 + CB))
        L = s.stop - s.start
        G = np.cumsum(g[s], 0)
        kb, qb, vb, bb = k[s], q[s], v[s], beta[s]
        E = np.exp(G[:, None, :] - G[None, :, :])
        A = np.tril(bb[:, None] * np.einsum("tc,jc,tjc->tj", kb, kb, E), -1)
        P = np.tril(np.einsum("tc,jc,tjc->tj", qb, kb, E))
        Ti = np.linalg.inv(np.eye(L) + A)
        U, W = Ti @ (bb[:, None] * vb), Ti @ (bb[:, None] * kb * np.exp(G))
        Dm = U - _mm(W, S.T, split)
        out[s] = _mm(qb * np.exp(G), S.T, split) + _mm(P, Dm, split)
        S = S * np.exp(G[-1])[None, :] + _mm(Dm.T, kb * np.exp(G[-1][None, :] - G), split)
    return out, S


def test_split_products_set_the_bf16x3_element_bar():
    """The block form equals the token-by-token definition (the oracle), and
    forming its state contractions with bf16-split operands (16 significant
    bits a product) leaves the per-unit error near 5e-6 while the worst
    element reaches about 1.3e-4 of its unit's rms over these nine sequences:
    on a sequence resumed from a random state an output element is a sum of
    about 190 such products of random sign.  That is the reading behind the element bar ELEM_TOL_SPLIT
    for fp32 tensors of the bf16x3 mode; the fp32 mode keeps 1e-4."""
    rng = np.random.default_rng(7)
    D = 128
    worst = 0.0
    for T in (320,) * 8 + (1024,):  # eight 5-block sequences and a 16-block one
        q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
        g = -np.log1p(np.exp(rng.standard_normal((T, D))))
        beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
        S0 = rng.standard_normal((D, D))
        pool = np.concatenate([np.zeros((1, 1, D, D)), S0[None, None]])
        one = np.array([1], np.int32)
        o_ref, p_ref = oracle.prefill(q[:, None], k[:, None], v[:, None], g[:, None],
                                      beta[:, None], np.array([0, T], np.int32), one, one, pool,
                                      kda=True, state_dtype="fp32", io_dtype="fp64")
        o_ref, s_ref = o_ref[:, 0], p_ref[1, 0]
        o64, s64 = _chunked(q, k, v, g, beta, S0, split=False)
        assert np.abs(o64 - o_ref).max() < 1e-12          # the block algebra is exact
        assert np.abs(s64 - s_ref).max() < 1e-7           # (the oracle rounds S to fp32)
        o, s = _chunked(q, k, v, g, beta, S0, split=True)
        unit = max(rel_err_units(o[None], o_ref[None], 1), rel_err_units(s[None], s_ref[None], 1))
        el = max(elem_err(o[None], o_ref[None], 1)[0], elem_err(s[None], s_ref[None], 1)[0])
        print(f"T={T}: split products, unit {unit:.2e}, element {el:.2e}")
        assert unit < 1e-5
        assert el < ELEM_TOL_SPLIT
        worst = max(worst, el)
    assert worst > TOL["fp32"]  # the split arithmetic itself misses 1e-4 per element
