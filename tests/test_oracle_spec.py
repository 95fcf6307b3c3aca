"""Pins of the oracle's speculative-decode functions (verify, exact commit,
conv-window scatter, state tracking) against the decode oracle, which the
pins in test_oracle_pins.py tie to closed forms and brute force.

Sources: the ReplaySSM passages of xxmr.cn/news/181459 (verify computes every
draft step's output from the checkpoint without writing the state back; the
ring records (d, k, g) and (rawv, rawk, g, beta) per step; the exact commit
replays the accepted prefix from the checkpoint; the fast-rebuild unrolled
sum), its "intermediate_conv_window" passage (per-step conv history, scattered
at the last accepted step) and its state-tracking passage (masked copy of the
conv and SSM rows from the active to the tracking slot).
"""
import numpy as np
import pytest

import oracle
from linear_attention_recurrent_amd import synth

EPS = 1e-6


def _case(seed, B, D, Hqk, Hv, d, kda, P=6):
    C = 2 * Hqk * d + Hv * d
    x = synth.normal(seed, synth.S_X, (B, D, C))
    w = 0.5 * synth.normal(seed, synth.S_W, (C, 4))
    g = synth.log_decay(seed, synth.S_G, (B, D, Hv, d) if kda else (B, D, Hv)).astype(np.float64)
    beta = synth.beta_gate(seed, synth.S_BETA, (B, D, Hv)).astype(np.float64)
    conv = synth.normal(seed, synth.S_CONV, (P + 1, 3, C))
    ssm = synth.normal(seed, synth.S_SSM, (P + 1, Hv, d, d))
    slots = synth.slot_permutation(seed, synth.S_SLOTS, P)[:B].astype(np.int32)
    return C, x, w, g, beta, conv, ssm, slots


def _sequential(x, w, g, beta, conv, ssm, slots, n, Hqk, Hv, d, kda):
    """n decode-oracle steps in fp64 (no rounding anywhere)."""
    outs, convs, states = [], [], []
    for t in range(n):
        o, conv, ssm = oracle.decode(x[:, t], w, None, conv, g[:, t], beta[:, t], slots, ssm,
                                     Hqk=Hqk, Hv=Hv, dk=d, dv=d, kda=kda, conv_dtype="fp64",
                                     state_dtype="fp64", io_dtype="fp64")
        outs.append(o)
        convs.append(conv.copy())
        states.append(ssm.copy())
    return outs, convs, states


@pytest.mark.parametrize("kda,Hqk,Hv", [(True, 2, 2), (False, 2, 4)])
def test_verify_equals_sequential_decode_and_commit_replays_it(kda, Hqk, Hv):
    B, D, d, L = 3, 5, 16, 8
    C, x, w, g, beta, conv, ssm, slots = _case(41, B, D, Hqk, Hv, d, kda)
    n_tok = np.array([D, D, D], np.int32)
    base = np.array([0, 5, 7], np.int32)  # positions wrap around the ring
    ring = oracle.new_ring(ssm.shape[0], Hv, L, d, d, kda)
    out, win, ring = oracle.verify(x, w, None, conv, g, beta, slots, n_tok, ssm, ring, base,
                                   Hqk=Hqk, Hv=Hv, dk=d, dv=d, kda=kda, conv_dtype="fp64",
                                   io_dtype="fp64")
    outs, convs, states = _sequential(x, w, g, beta, conv, ssm, slots, D, Hqk, Hv, d, kda)
    for t in range(D):
        np.testing.assert_array_equal(out[:, t], outs[t])
        np.testing.assert_array_equal(win[:, t], convs[t][slots])
    for a in range(D + 1):
        acc = np.full(B, a, np.int32)
        new = oracle.commit(acc, slots, ssm, ring, base, kda=kda, state_dtype="fp64")
        want = ssm if a == 0 else states[a - 1]
        np.testing.assert_array_equal(new[slots], want[slots])
        others = np.setdiff1d(np.arange(ssm.shape[0]), slots)
        np.testing.assert_array_equal(new[others], ssm[others])


def test_ring_records_rebuild_the_state_by_the_unrolled_sum():
    """The ring's (d, k, g) reproduce S_m = S_0 Diag(prod alpha) +
    sum_j d_j (k_j . prod_{i>j} alpha_i)^T, and k = rawk / sqrt(|rawk|^2 + eps)."""
    B, D, Hqk, Hv, d, L = 2, 6, 1, 1, 16, 8
    C, x, w, g, beta, conv, ssm, slots = _case(42, B, D, Hqk, Hv, d, True)
    base = np.array([3, 6], np.int32)
    ring = oracle.new_ring(ssm.shape[0], Hv, L, d, d, True)
    _, _, ring = oracle.verify(x, w, None, conv, g, beta, slots, [D, D], ssm, ring, base,
                               Hqk=Hqk, Hv=Hv, dk=d, dv=d, conv_dtype="fp64", io_dtype="fp64")
    _, _, states = _sequential(x, w, g, beta, conv, ssm, slots, D, Hqk, Hv, d, True)
    for b, s in enumerate(slots):
        pos = [(base[b] + t) % L for t in range(D)]
        ks, ds, gs = ring["k"][s, 0, pos], ring["d"][s, 0, pos], ring["g"][s, 0, pos]
        np.testing.assert_allclose(ks, ring["rawk"][s, 0, pos] / np.sqrt(
            np.sum(ring["rawk"][s, 0, pos] ** 2, axis=1, keepdims=True) + EPS), rtol=1e-14)
        for m in range(1, D + 1):
            S = ssm[s, 0] * np.exp(gs[:m].sum(0))[None, :]
            for j in range(m):
                S = S + np.outer(ds[j], ks[j] * np.exp(gs[j + 1:m].sum(0)))
            np.testing.assert_allclose(S, states[m - 1][s, 0], rtol=1e-11, atol=1e-12)


def test_partial_drafts_and_conv_scatter_at_the_last_accepted_step():
    B, D, Hqk, Hv, d, L = 3, 4, 1, 1, 16, 8
    C, x, w, g, beta, conv, ssm, slots = _case(43, B, D, Hqk, Hv, d, True)
    n_tok = np.array([4, 2, 0], np.int32)
    ring = oracle.new_ring(ssm.shape[0], Hv, L, d, d, True)
    out, win, ring = oracle.verify(x, w, None, conv, g, beta, slots, n_tok, ssm, ring,
                                   [0, 0, 0], Hqk=Hqk, Hv=Hv, dk=d, dv=d, conv_dtype="fp64",
                                   io_dtype="fp64")
    assert np.all(out[1, 2:] == 0) and np.all(out[2] == 0)
    _, convs, _ = _sequential(x, w, g, beta, conv, ssm, slots, D, Hqk, Hv, d, True)
    accepted = np.array([3, 2, 0], np.int32)
    mask = np.array([1, 1, 0], bool)
    new_conv = oracle.conv_window_scatter(conv, win, mask, slots, accepted - 1)
    for b in range(2):
        np.testing.assert_array_equal(new_conv[slots[b]], convs[accepted[b] - 1][slots[b]])
    np.testing.assert_array_equal(new_conv[slots[2]], conv[slots[2]])


def test_bf16_io_rounds_the_conv_output_and_the_ring_replays_it():
    """With bf16 I/O the conv output is stored rounded (as a separate conv
    kernel would), verify runs on those values, and the ring keeps them: verify
    equals decode steps fed the bf16-rounded conv output, and the commit of a
    steps reproduces the state of a such steps exactly."""
    B, D, Hqk, Hv, d, L = 2, 4, 1, 2, 16, 8
    C, x, w, g, beta, conv, ssm, slots = _case(44, B, D, Hqk, Hv, d, True)
    x = oracle.round_to(x, "bf16")
    conv = oracle.round_to(conv, "bf16")
    ring = oracle.new_ring(ssm.shape[0], Hv, L, d, d, True)
    out, win, ring = oracle.verify(x, w, None, conv, g, beta, slots, [D, D], ssm, ring, [0, 0],
                                   Hqk=Hqk, Hv=Hv, dk=d, dv=d, conv_dtype="bf16",
                                   io_dtype="bf16")
    cpool, spool = conv, ssm
    for t in range(D):
        y, cpool = oracle.shortconv_step(x[:, t], w, None, cpool, slots, conv_dtype="bf16")
        o, _, spool = oracle.decode(oracle.round_to(y, "bf16"), None, None, None, g[:, t],
                                    beta[:, t], slots, spool, Hqk=Hqk, Hv=Hv, dk=d, dv=d,
                                    state_dtype="fp64", io_dtype="fp64")
        np.testing.assert_array_equal(out[:, t], oracle.round_to(o, "bf16"))
        np.testing.assert_array_equal(win[:, t], cpool[slots])
        new = oracle.commit(np.full(B, t + 1, np.int32), slots, ssm, ring, [0, 0], kda=True,
                            state_dtype="fp64")
        np.testing.assert_array_equal(new[slots], spool[slots])
    assert np.array_equal(ring["rawk"], oracle.round_to(ring["rawk"], "bf16"))
    assert np.array_equal(ring["d"], oracle.round_to(ring["d"], "bf16"))


def test_track_copy_copies_masked_rows_only():
    conv = synth.normal(45, 0, (6, 3, 10))
    ssm = synth.normal(45, 1, (6, 2, 4, 4))
    new_conv, new_ssm = oracle.track_copy(conv, ssm, [1, 0, 1], [1, 2, 3], [4, 5, 3])
    np.testing.assert_array_equal(new_conv[4], conv[1])
    np.testing.assert_array_equal(new_ssm[4], ssm[1])
    np.testing.assert_array_equal(new_conv[5], conv[5])   # masked off
    np.testing.assert_array_equal(new_ssm[[0, 1, 2, 3, 5]], ssm[[0, 1, 2, 3, 5]])


@pytest.mark.parametrize("kda", [True, False])
def test_ring_fold_equals_the_exact_commit_on_exact_records(kda):
    """With fp64 records the fast rebuild's unrolled sum and the exact replay
    of the same steps give the same state; m = 0 copies the checkpoint; the
    projection is scale S_m q_hat."""
    B, D, Hqk, Hv, d, L = 3, 6, 1, 2, 16, 8
    C, x, w, g, beta, conv, ssm, slots = _case(46 + kda, B, D, Hqk, Hv, d, kda)
    base = np.array([5, 0, 3], np.int32)
    ring = oracle.new_ring(ssm.shape[0], Hv, L, d, d, kda)
    _, _, ring = oracle.verify(x, w, None, conv, g, beta, slots, [D] * B, ssm, ring, base,
                               Hqk=Hqk, Hv=Hv, dk=d, dv=d, kda=kda, conv_dtype="fp64",
                               io_dtype="fp64")
    m = np.array([6, 2, 0], np.int32)
    exact = oracle.commit(m, slots, ssm, ring, base, kda=kda, state_dtype="fp64")
    dst = np.array([slots[0], 0, slots[2]], np.int32)   # one to another row
    q = synth.normal(48, 0, (B, Hv, d))
    fold, out = oracle.ring_fold(m, slots, dst, ssm, ring, base, q, kda=kda, state_dtype="fp64",
                                 io_dtype="fp64", scale=0.5)
    np.testing.assert_allclose(fold[slots[0]], exact[slots[0]], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fold[0], exact[slots[1]], rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(fold[slots[2]], ssm[slots[2]])
    qh = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + EPS)
    for b, s in enumerate(dst):
        for h in range(Hv):
            np.testing.assert_allclose(out[b, h], 0.5 * fold[s, h] @ qh[b, h], rtol=1e-12,
                                       atol=1e-13)
