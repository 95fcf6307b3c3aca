"""GPU parity of the speculative-decode entry points (verify, exact commit,
conv-window scatter, state-tracking copy) against the fp64 oracle, through the
C ABI.

Bars: every step's output, the ring's vectors and the committed state within
the relative-L2 tolerance of their storage dtype (1e-4 fp32, 2e-2 bf16) per
(request, step, head) or (request, head); conv windows, the ring's gates, the
scattered conv rows, the tracking copies and every untouched pool row
bit-exact.  Verify has two forms: up to 8 draft tokens the chunk form (one
matrix-core product with the checkpoint), beyond that the sequential form;
both are checked against the oracle; so are the commit's two forms (up to 8
accepted steps the chunk form, beyond that the sequential replay).
Committing a verify's first steps and verifying the rest from the committed
state reproduces the first call's later outputs: bit for bit when every call
takes the sequential form (they run the same per-row arithmetic), within the
fp32 bar in the chunk form.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_amd import binding as la
from linear_attention_recurrent_amd import synth
from parity_util import TOL, assert_close_units, f64

pytestmark = pytest.mark.gpu

D_HEAD = 128


def make_case(seed, B, D, Hqk, Hv, kda, io, state, conv, P, dev, L=16):
    d = D_HEAD
    C = 2 * Hqk * d + Hv * d
    x = synth.to_torch(synth.normal(seed, synth.S_X, (B, D, C)), io, dev)
    w = synth.to_torch(0.5 * synth.normal(seed, synth.S_W, (C, 4)), "fp32", dev)
    g = torch.from_numpy(synth.log_decay(seed, synth.S_G, (B, D, Hv, d) if kda else (B, D, Hv))).to(dev)
    beta = torch.from_numpy(synth.beta_gate(seed, synth.S_BETA, (B, D, Hv))).to(dev)
    conv_pool = synth.to_torch(synth.normal(seed, synth.S_CONV, (P + 1, 3, C)), conv, dev)
    ssm_pool = synth.to_torch(synth.normal(seed, synth.S_SSM, (P + 1, Hv, d, d)), state, dev)
    slots = torch.from_numpy(synth.slot_permutation(seed, synth.S_SLOTS, P)[:B].astype(np.int32)).to(dev)
    ring = la.new_ring(P + 1, Hv, L, d, d, kda=kda, dtype=x.dtype, device=dev)
    return dict(x=x, w=w, g=g, beta=beta, conv_pool=conv_pool, ssm_pool=ssm_pool, slots=slots,
                ring=ring, C=C)


def i32(v, dev):
    return torch.tensor(v, dtype=torch.int32, device=dev)


def run_verify(kda, c, n_tok, base, Hqk, dev):
    fn = la.kda_verify if kda else la.gdn_verify
    return fn(c["x"], c["g"], c["beta"], c["slots"], i32(n_tok, dev), c["ssm_pool"], c["ring"],
              i32(base, dev), Hqk=Hqk, conv_w=c["w"], conv_pool=c["conv_pool"])


def oracle_verify(kda, c, n_tok, base, Hqk, Hv, io, conv):
    return oracle.verify(f64(c["x"]), f64(c["w"]), None, f64(c["conv_pool"]), f64(c["g"]),
                         f64(c["beta"]), c["slots"].cpu().numpy(), n_tok, f64(c["ssm_pool"]),
                         oracle.new_ring(c["ssm_pool"].shape[0], Hv, c["ring"]["d"].shape[2],
                                         D_HEAD, D_HEAD, kda), base, Hqk=Hqk, Hv=Hv,
                         dk=D_HEAD, dv=D_HEAD, kda=kda, conv_dtype=conv, io_dtype=io)


CASES = [  # kda, Hqk, Hv, io, state, conv
    (True, 2, 2, "bf16", "bf16", "bf16"),
    (True, 2, 2, "fp32", "fp32", "fp32"),
    (True, 1, 2, "bf16", "fp32", "bf16"),
    (False, 2, 4, "fp32", "fp32", "fp32"),
    (False, 2, 4, "bf16", "bf16", "fp32"),
]


@pytest.mark.parametrize("D", [8, 12])   # the chunk form, the sequential form
@pytest.mark.parametrize("kda,Hqk,Hv,io,state,conv", CASES)
def test_verify_and_commit_match_oracle(kda, Hqk, Hv, io, state, conv, D, dev):
    B, P = 4, 10
    c = make_case(7100 + Hv + 10 * kda + D, B, D, Hqk, Hv, kda, io, state, conv, P, dev)
    n_tok = [D, 5, 1, 0]
    base = [0, 13, 7, 3]                      # wraps around the 16-deep ring
    conv0, ssm0 = c["conv_pool"].clone(), c["ssm_pool"].clone()
    out, win = run_verify(kda, c, n_tok, base, Hqk, dev)
    torch.cuda.synchronize()
    o_ref, w_ref, r_ref = oracle_verify(kda, c, n_tok, base, Hqk, Hv, io, conv)
    assert torch.equal(c["conv_pool"], conv0) and torch.equal(c["ssm_pool"], ssm0)
    assert_close_units(f64(out), o_ref, 3, io, "verify outputs")
    assert np.all(f64(out)[1, 5:] == 0) and np.all(f64(out)[3] == 0)
    slots = c["slots"].cpu().numpy()
    ring = {k: f64(v) for k, v in c["ring"].items()}
    for b in range(B):
        s = slots[b]
        pos = [(base[b] + t) % 16 for t in range(n_tok[b])]
        if not pos:
            continue
        np.testing.assert_array_equal(f64(win)[b, :n_tok[b]], w_ref[b, :n_tok[b]])
        for key in ("g", "beta"):  # (GDN's g is [rows, Hv, L] here, [rows, Hv, L, 1] there)
            want = r_ref[key][s][:, pos]
            np.testing.assert_array_equal(ring[key][s][:, pos].reshape(want.shape), want)
        for key in ("d", "k", "rawv", "rawk"):
            assert_close_units(ring[key][s][:, pos], r_ref[key][s][:, pos], 2, io, f"ring {key}")

    accepted = [6 if D <= 8 else 10, 3, 1, 0]   # 10: the sequential commit, the rest the chunk form
    fn = la.kda_commit if kda else la.gdn_commit
    fn(i32(accepted, dev), c["slots"], c["ssm_pool"], c["ring"], i32(base, dev))
    torch.cuda.synchronize()
    p_ref = oracle.commit(accepted, slots, f64(ssm0), ring, base, kda=kda, state_dtype=state)
    got = f64(c["ssm_pool"])
    assert_close_units(got[slots[:3]], p_ref[slots[:3]], 2, state, "committed state")
    untouched = np.setdiff1d(np.arange(P + 1), slots[:3])
    np.testing.assert_array_equal(got[untouched], f64(ssm0)[untouched])


def continue_after_commit(D, a, io, dev, L=16):
    """fp32 state: verify D tokens; commit a and scatter the conv window of
    step a - 1; verify the remaining D - a tokens from the committed pools.
    Returns the first call's outputs of steps a.. and the second call's."""
    B, Hqk, Hv, P = 3, 2, 2, 8
    c = make_case(7200 + D, B, D, Hqk, Hv, True, io, "fp32", "bf16", P, dev, L=L)
    out1, win1 = run_verify(True, c, [D] * B, [0] * B, Hqk, dev)
    la.kda_commit(i32([a] * B, dev), c["slots"], c["ssm_pool"], c["ring"], i32([0] * B, dev))
    la.conv_window_scatter(win1, c["slots"], i32([a - 1] * B, dev), c["conv_pool"])
    c2 = dict(c, x=c["x"][:, a:].contiguous(), g=c["g"][:, a:].contiguous(),
              beta=c["beta"][:, a:].contiguous())
    out2, _ = run_verify(True, c2, [D - a] * B, [a] * B, Hqk, dev)
    torch.cuda.synchronize()
    return out1[:, a:], out2


def test_commit_then_verify_continues_bit_exactly_sequential(dev):
    """20 tokens, commit 10, then 10 more (ring depth 32): both verifies and
    the commit take the sequential form, whose steps run the same per-row
    arithmetic, so the outputs agree bit for bit."""
    first, second = continue_after_commit(20, 10, "bf16", dev, L=32)
    assert torch.equal(second, first)


def test_commit_then_verify_continues_chunk_form(dev):
    """5 tokens, commit 3, then 2 more, fp32 I/O: the verifies and the commit
    take the chunk form; the continuation agrees with the first call within
    the fp32 bar."""
    first, second = continue_after_commit(5, 3, "fp32", dev)
    assert_close_units(f64(second), f64(first), 2, "fp32", "continued outputs")


@pytest.mark.parametrize("kda", [True, False])
def test_chunk_forms_at_extreme_decays(kda, dev):
    """The chunk forms of verify and commit where the decay is extreme: no
    decay at all (g = 0), a decay strong enough to underflow exp(G) within
    the chunk (g = -30 per step), and the two alternating per channel (KDA)
    or per step (GDN).  Every exponent the chunk form takes is <= 0, so
    nothing overflows; outputs, ring d and the committed state stay within
    the fp32 bar of the oracle."""
    B, D, Hqk, Hv, P = 3, 8, 2, 2, 6
    c = make_case(7600 + kda, B, D, Hqk, Hv, kda, "fp32", "fp32", "fp32", P, dev)
    shape = c["g"].shape
    g = torch.zeros(shape, dtype=torch.float32)
    g[1] = -30.0                                       # request 1: strong decay
    if kda:
        g[2, :, :, 1::2] = -30.0                       # request 2: alternating channels
    else:
        g[2, 1::2] = -30.0                             # request 2: alternating steps
    c["g"] = g.to(dev)
    n_tok, base = [D, D, D], [0, 5, 11]
    ssm0 = c["ssm_pool"].clone()
    out, _ = run_verify(kda, c, n_tok, base, Hqk, dev)
    torch.cuda.synchronize()
    o_ref, _, r_ref = oracle_verify(kda, c, n_tok, base, Hqk, Hv, "fp32", "fp32")
    assert np.all(np.isfinite(f64(out)))
    assert_close_units(f64(out), o_ref, 3, "fp32", "verify outputs")
    slots = c["slots"].cpu().numpy()
    ring = {k: f64(v) for k, v in c["ring"].items()}
    for b in range(B):
        pos = [(base[b] + t) % 16 for t in range(D)]
        assert_close_units(ring["d"][slots[b]][:, pos], r_ref["d"][slots[b]][:, pos], 2, "fp32", "ring d")
    accepted = [8, 8, 5]
    fn = la.kda_commit if kda else la.gdn_commit
    fn(i32(accepted, dev), c["slots"], c["ssm_pool"], c["ring"], i32(base, dev))
    torch.cuda.synchronize()
    p_ref = oracle.commit(accepted, slots, f64(ssm0), ring, base, kda=kda, state_dtype="fp32")
    got = f64(c["ssm_pool"])
    assert np.all(np.isfinite(got))
    assert_close_units(got[slots], p_ref[slots], 2, "fp32", "committed state")


@pytest.mark.parametrize("kda", [1, 0], ids=["kda", "gdn"])
def test_chunk_forms_with_a_full_reset(kda, dev):
    """A gate of -inf empties the state at that step (exp(-inf) = 0), so the
    outputs after it depend on the later steps only.  The chunk forms of
    verify and commit, and the fold, take differences of running gate sums;
    the reset must not turn those into NaN.  Request 0 resets mid-chunk, request 1 at its
    first step, request 2 at its last step; for KDA request 0 resets only the
    even key channels."""
    B, D, Hqk, Hv, P = 3, 8, 2, 2, 6
    c = make_case(7700 + kda, B, D, Hqk, Hv, kda, "fp32", "fp32", "fp32", P, dev)
    g = c["g"].cpu().clone()
    if kda:
        g[0, 3, :, 0::2] = float("-inf")
        g[1, 0] = float("-inf")
        g[2, D - 1] = float("-inf")
    else:
        g[0, 3] = float("-inf")
        g[1, 0] = float("-inf")
        g[2, D - 1] = float("-inf")
    c["g"] = g.to(dev)
    n_tok, base = [D, D, D], [0, 5, 11]
    ssm0 = c["ssm_pool"].clone()
    out, _ = run_verify(kda, c, n_tok, base, Hqk, dev)
    torch.cuda.synchronize()
    o_ref, _, r_ref = oracle_verify(kda, c, n_tok, base, Hqk, Hv, "fp32", "fp32")
    assert np.all(np.isfinite(f64(out)))
    assert_close_units(f64(out), o_ref, 3, "fp32", "verify outputs")
    slots = c["slots"].cpu().numpy()
    ring = {k: f64(v) for k, v in c["ring"].items()}
    for b in range(B):
        pos = [(base[b] + t) % 16 for t in range(D)]
        assert_close_units(ring["d"][slots[b]][:, pos], r_ref["d"][slots[b]][:, pos], 2, "fp32", "ring d")
    accepted = [6, 8, 8]
    fn = la.kda_commit if kda else la.gdn_commit
    fn(i32(accepted, dev), c["slots"], c["ssm_pool"], c["ring"], i32(base, dev))
    torch.cuda.synchronize()
    p_ref = oracle.commit(accepted, slots, f64(ssm0), ring, base, kda=kda, state_dtype="fp32")
    got = f64(c["ssm_pool"])
    assert np.all(np.isfinite(got))
    assert_close_units(got[slots], p_ref[slots], 2, "fp32", "committed state")
    # the fast rebuild of the same records, from the checkpoint
    pool = ssm0.clone()
    q = synth.to_torch(synth.normal(7701, 0, (B, Hv, D_HEAD)), "fp32", dev)
    m = [8, 8, 6]
    ffn = la.kda_ring_fold if kda else la.gdn_ring_fold
    out = ffn(i32(m, dev), c["slots"], pool, c["ring"], i32(base, dev), q=q)
    torch.cuda.synchronize()
    f_ref, fo_ref = oracle.ring_fold(m, slots, slots, f64(ssm0), ring, base, f64(q), kda=kda,
                                     state_dtype="fp32", io_dtype="fp32", scale=1.0)
    got = f64(pool)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(f64(out)))
    assert_close_units(got[slots], f_ref[slots], 2, "fp32", "folded state")
    assert_close_units(f64(out), fo_ref, 2, "fp32", "fold projection")


def test_conv_window_scatter_and_track_copy_are_bit_exact(dev):
    B, D, C, P = 5, 4, 768, 12
    conv = synth.to_torch(synth.normal(7300, 0, (P + 1, 3, C)), "bf16", dev)
    ssm = synth.to_torch(synth.normal(7300, 1, (P + 1, 2, D_HEAD, D_HEAD)), "fp32", dev)
    windows = synth.to_torch(synth.normal(7300, 2, (B, D, 3, C)), "bf16", dev)
    slots = [3, 7, 1, 9, 4]
    step = [0, 3, 2, -1, 1]                   # -1: nothing accepted
    mask = torch.tensor([1, 1, 0, 1, 1], dtype=torch.uint8, device=dev)
    ref = oracle.conv_window_scatter(f64(conv), f64(windows), mask.cpu().numpy(), slots, step)
    la.conv_window_scatter(windows, i32(slots, dev), i32(step, dev), conv, mask=mask)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(conv), ref)

    src, dst = [1, 2, 3, 5], [10, 11, 3, 12]  # one self-copy
    tmask = torch.tensor([1, 1, 1, 0], dtype=torch.uint8, device=dev)
    ref_c, ref_s = oracle.track_copy(f64(conv), f64(ssm), tmask.cpu().numpy(), src, dst)
    la.state_track_copy(i32(src, dev), i32(dst, dev), conv, ssm, mask=tmask)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(conv), ref_c)
    np.testing.assert_array_equal(f64(ssm), ref_s)


def test_verify_full_shape_kda_64x12_bf16(dev):
    """The serving shape of one layer (64 requests, 12 heads, bf16) with 8
    draft tokens, every request and step against the oracle, then the commit
    of a per-request accepted count."""
    B, D, H, P = 64, 8, 12, 80
    c = make_case(7400, B, D, H, H, True, "bf16", "bf16", "bf16", P, dev)
    rng = np.random.default_rng(7400)
    n_tok = [D] * B
    base = rng.integers(0, 16, B).tolist()
    ssm0 = c["ssm_pool"].clone()
    out, win = run_verify(True, c, n_tok, base, H, dev)
    torch.cuda.synchronize()
    o_ref, w_ref, _ = oracle_verify(True, c, n_tok, base, H, H, "bf16", "bf16")
    assert_close_units(f64(out), o_ref, 3, "bf16", "verify outputs")
    np.testing.assert_array_equal(f64(win), w_ref)
    accepted = rng.integers(0, D + 1, B).tolist()
    la.kda_commit(i32(accepted, dev), c["slots"], c["ssm_pool"], c["ring"], i32(base, dev))
    torch.cuda.synchronize()
    ring = {k: f64(v) for k, v in c["ring"].items()}
    slots = c["slots"].cpu().numpy()
    p_ref = oracle.commit(accepted, slots, f64(ssm0), ring, base, kda=True, state_dtype="bf16")
    assert_close_units(f64(c["ssm_pool"])[slots], p_ref[slots], 2, "bf16", "committed state")


FOLD_CASES = [  # kda, Hqk, Hv, io, state, L, D
    (True, 2, 2, "bf16", "bf16", 16, 8),
    (True, 1, 2, "fp32", "fp32", 32, 20),     # two LDS passes (16 + 4 steps)
    (False, 2, 4, "bf16", "fp32", 16, 8),
]


@pytest.mark.parametrize("kda,Hqk,Hv,io,state,L,D", FOLD_CASES)
def test_ring_fold_matches_oracle(kda, Hqk, Hv, io, state, L, D, dev):
    """The fast rebuild of the ring a verify wrote, against the oracle's
    unrolled sum on the same records: state (in place and to another row)
    and the projection scale S_m q_hat."""
    B, P = 4, 10
    c = make_case(7500 + Hv + L, B, D, Hqk, Hv, kda, io, state, "bf16", P, dev, L=L)
    base = [0, L - 3, 5, 1]
    run_verify(kda, c, [D] * B, base, Hqk, dev)
    ssm0 = c["ssm_pool"].clone()
    slots = c["slots"].cpu().numpy()
    m = [D, 3, 0, 5]
    dst = [int(slots[0]), 0, int(slots[2]), int(slots[3])]   # entry 1 folds into row 0
    q = synth.to_torch(synth.normal(7501, 0, (B, Hv, D_HEAD)), io, dev)
    fn = la.kda_ring_fold if kda else la.gdn_ring_fold
    out = fn(i32(m, dev), c["slots"], c["ssm_pool"], c["ring"], i32(base, dev), dst=i32(dst, dev),
             q=q, scale=0.75)
    torch.cuda.synchronize()
    ring = {k: f64(v) for k, v in c["ring"].items()}
    p_ref, o_ref = oracle.ring_fold(m, slots, dst, f64(ssm0), ring, base, f64(q), kda=kda,
                                    state_dtype=state, io_dtype=io, scale=0.75)
    got = f64(c["ssm_pool"])
    assert_close_units(got[dst], p_ref[dst], 2, state, "folded state")
    assert_close_units(f64(out), o_ref, 2, io, "projection")
    untouched = np.setdiff1d(np.arange(P + 1), dst)
    np.testing.assert_array_equal(got[untouched], f64(ssm0)[untouched])
    if io == "fp32":  # exact fp32 records: the fold agrees with the exact replay
        exact = oracle.commit(m, slots, f64(ssm0), ring, base, kda=kda, state_dtype="fp64")
        for b in (0, 3):
            assert_close_units(got[dst[b]], exact[slots[b]], 1, "fp32", "fold vs exact commit")


def test_graph_replay_verify_commit_matches_eager(dev):
    """Verify then commit (chunk forms, bf16) captured in one HIP graph and
    replayed several times, each replay committing onto the state the last
    one left, with eager work between replays: bit-identical to eager calls
    at every replay."""
    B, D, Hqk, Hv, P = 4, 8, 2, 2, 6
    c = make_case(7800, B, D, Hqk, Hv, 1, "bf16", "bf16", "bf16", P, dev)
    cb = dict(c, ssm_pool=c["ssm_pool"].clone(), conv_pool=c["conv_pool"].clone(),
              ring={k: v.clone() for k, v in c["ring"].items()})
    n_tok, base, acc = i32([D] * B, dev), i32([0, 3, 8, 5], dev), i32([8, 5, 1, 8], dev)
    outs = {}

    def call(cc, key):
        outs[key] = la.kda_verify(cc["x"], cc["g"], cc["beta"], cc["slots"], n_tok, cc["ssm_pool"],
                                  cc["ring"], base, Hqk=Hqk, conv_w=cc["w"],
                                  conv_pool=cc["conv_pool"], out=outs.get(key))[0]
        la.kda_commit(acc, cc["slots"], cc["ssm_pool"], cc["ring"], base)

    call(cb, "b")   # warm-up outside capture
    call(c, "a")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cb, "b")
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        call(c, "a")
        torch.cuda.synchronize()
        assert torch.equal(outs["a"], outs["b"]), rep
        assert torch.equal(c["ssm_pool"], cb["ssm_pool"]), rep
        for k in c["ring"]:
            assert torch.equal(c["ring"][k], cb["ring"][k]), (rep, k)
