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
from parity_util import elem_err, rel_err_units


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
