"""GPU parity of the prefill path against the fp64 oracle, through the C ABI:
the varlen short conv (history hand-off through conv-pool slots) and the
chunked KDA / GDN prefill (blocks of 64 tokens, initial state from slot_in,
final state to slot_out).

Bars: conv-state contents bit-exact; outputs and states within the relative
L2 tolerance of their storage dtype per (sequence or token, head); packing
sequences that start on 64-token boundaries is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_amd import binding as la
from linear_attention_recurrent_amd import synth
from parity_util import assert_close_seqs, assert_close_units, elem_tol, f64

pytestmark = pytest.mark.gpu

D = 128


def prefill_case(lens, Hqk, Hv, seed, dev, *, kda=True, io="bf16", state="fp32",
                 slot_in=None, slot_out=None, P=None):
    sh = synth.PrefillShape(seqlens=tuple(lens), Hqk=Hqk, Hv=Hv, dk=D, dv=D, kda=kda, io=io,
                            state=state)
    inp = synth.prefill_inputs(sh, seed, dev)
    N = len(lens)
    P = P or (2 * N + 2)
    pool = synth.normal_torch(seed, synth.S_SSM, (P + 1) * Hv * D * D, dev,
                              synth.TORCH_DTYPE[state]).view(P + 1, Hv, D, D)
    si = np.array(slot_in if slot_in is not None else [-1] * N, dtype=np.int32)
    so = np.array(slot_out if slot_out is not None else list(range(1, N + 1)), dtype=np.int32)
    return sh, inp, pool, si, so


def run_gpu(sh, inp, pool, si, so, **kw):
    fn = la.kda_prefill_chunked if sh.kda else la.gdn_prefill_chunked
    dev = pool.device
    return fn(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
              torch.from_numpy(si).to(dev), torch.from_numpy(so).to(dev), pool, **kw)


def run_oracle(sh, inp, pool, si, so, heads=None):
    """Oracle on all heads, or on a subset of value heads.  A sampled value
    head h takes its q/k head h // (Hv / Hqk) along, so the oracle runs the
    subset with one q/k head per value head."""
    q, k, v, g, beta = (f64(inp[x]) for x in ("q", "k", "v", "g", "beta"))
    p = f64(pool)
    if heads is not None:
        kh = [h // (sh.Hv // sh.Hqk) for h in heads]
        q, k = q[:, kh], k[:, kh]
        v, g, beta = v[:, heads], g[:, heads], beta[:, heads]
        p = p[:, heads]
    return oracle.prefill(q, k, v, g, beta, inp["cu_seqlens"].cpu().numpy(), si, so, p,
                          kda=sh.kda, state_dtype=sh.state, io_dtype=sh.io)


MODES = {"fp32": la.LA_PREFILL_FP32, "bf16x3": la.LA_PREFILL_BF16X3}


def check(sh, inp, pool, si, so, heads=None, what="", mode=la.LA_PREFILL_FP32):
    before = pool.clone()
    o_ref, p_ref = run_oracle(sh, inp, before, si, so, heads)
    out = run_gpu(sh, inp, pool, si, so, mode=mode)
    torch.cuda.synchronize()
    o = f64(out)
    p = f64(pool)
    if heads is not None:
        o, p = o[:, heads], p[:, heads]
    # outputs per (sequence, head); states per (slot, head).  Both precision
    # modes are held to the bar of the tensor's storage dtype, the split
    # products of bf16x3 mode to the derived element bar for fp32 tensors
    split = mode == la.LA_PREFILL_BF16X3
    assert_close_seqs(o, o_ref, inp["cu_seqlens"].cpu().numpy(), sh.io, f"{what} outputs",
                      etol=elem_tol(sh.io, split))
    assert_close_units(p[so], p_ref[so], 2, sh.state, f"{what} final states",
                       etol=elem_tol(sh.state, split))
    untouched = np.setdiff1d(np.arange(pool.shape[0]), so)
    assert np.array_equal(f64(pool)[untouched], f64(before)[untouched])
    return out


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("io,state", [("bf16", "fp32"), ("fp32", "fp32"), ("bf16", "bf16")])
def test_kda_prefill_varlen_matches_oracle(io, state, mode, dev):
    lens = [5, 64, 70, 1, 130, 3]
    N = len(lens)
    si = [-1, 7, -1, 8, 9, -1]             # fresh and resumed sequences
    so = [1, 7, 2, 3, 4, 5]                # slot_in == slot_out for one of them
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3000, dev, io=io, state=state, slot_in=si,
                                         slot_out=so, P=10)
    print(f"[prefill parity] kda io={io} state={state} mode={mode} lens={lens}", flush=True)
    check(sh, inp, pool, si, so, what=f"kda {io}/{state}/{mode}", mode=MODES[mode])


@pytest.mark.parametrize("mode", list(MODES))
def test_gdn_prefill_gqa_matches_oracle(mode, dev):
    lens = [100, 17, 64]
    sh, inp, pool, si, so = prefill_case(lens, 1, 2, 3001, dev, kda=False, io="fp32",
                                         state="fp32", slot_in=[2, -1, 3], slot_out=[4, 5, 6],
                                         P=7)
    check(sh, inp, pool, si, so, what=f"gdn gqa {mode}", mode=MODES[mode])


def test_kda_prefill_gqa_matches_oracle(dev):
    lens = [65, 40]
    sh, inp, pool, si, so = prefill_case(lens, 2, 4, 3002, dev, slot_in=[1, -1], slot_out=[2, 3],
                                         P=4)
    check(sh, inp, pool, si, so, what="kda gqa")


def test_empty_and_single_token_sequences(dev):
    lens = [0, 1, 0, 2, 63]
    sh, inp, pool, si, so = prefill_case(lens, 1, 1, 3003, dev, slot_in=[3, -1, 4, -1, -1],
                                         slot_out=[5, 6, 7, 8, 9], P=9)
    before = pool.clone()
    check(sh, inp, pool, si, so, what="empty/short")
    # an empty sequence hands its initial state over unchanged
    assert torch.equal(pool[5], before[3])
    assert torch.equal(pool[7], before[4])


@pytest.mark.parametrize("N,H", [(511, 1), (600, 1), (600, 24)])
def test_sequence_table_edge_and_global_search(N, H, dev):
    """Kernel 1 stages cu_seqlens and slot_in in LDS for fewer than 512
    sequences (511 fills the table) and searches cu_seqlens in global memory
    beyond (600).  Seeded lengths of 0-3 tokens put dozens of pieces in a
    tile; every other sequence resumes from a pool slot.  With 24 heads there
    are more (tile, head) items than workgroups, so consecutive items of one
    tile share a lookup, also on the global path."""
    rng = np.random.default_rng(3300 + N)
    lens = [int(x) for x in rng.integers(0, 4, size=N)]
    si = [n + 1 if n % 2 else -1 for n in range(N)]
    so = [N + 1 + n for n in range(N)]
    sh, inp, pool, si, so = prefill_case(lens, H, H, 3300 + N, dev, slot_in=si, slot_out=so,
                                         P=2 * N + 1)
    print(f"[prefill parity] {N} sequences, {H} heads, T={sum(lens)}", flush=True)
    check(sh, inp, pool, si, so, what=f"{N} sequences {H} heads", mode=la.LA_PREFILL_BF16X3)


@pytest.mark.parametrize("io,state", [("bf16", "fp32"), ("fp32", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
def test_items_across_tiles_with_four_value_heads_per_qk_head(kda, mode, io, state, dev):
    """More (tile, head) items than the persistent grid has workgroups
    (40 to 46 tiles x 8 value heads), so a workgroup walks more than one item and
    its range starts and ends inside a tile; the heads of a tile share the
    sequence lookup, refreshed where the tile changes.  Four value heads
    share each of the two q/k heads.  The 128 (sequence, head) pairs take
    the chain's 64-row form in bf16x3 mode, here with every dtype pairing of
    its state load, split and store."""
    rng = np.random.default_rng(3400 + kda)
    lens = [int(x) for x in rng.integers(1, 300, size=16)]
    N = len(lens)
    si = [n + 1 if n % 3 == 0 else -1 for n in range(N)]
    so = [N + 1 + n for n in range(N)]
    sh, inp, pool, si, so = prefill_case(lens, 2, 8, 3400 + kda, dev, kda=kda, io=io, state=state,
                                         slot_in=si, slot_out=so, P=2 * N + 1)
    print(f"[prefill parity] kda={kda} mode={mode} io={io} state={state} {N} sequences, "
          f"T={sum(lens)}, 2/8 heads", flush=True)
    check(sh, inp, pool, si, so, what=f"items across tiles kda={kda} {mode} {io}/{state}",
          mode=MODES[mode])


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
def test_strong_decay_diagonal_factorisation(mode, dev):
    """Log decays near -4 per token (16-token spread ~64, inside the
    exponent clamp) still match the oracle."""
    lens = [96]
    sh, inp, pool, si, so = prefill_case(lens, 1, 1, 3004, dev, io="fp32", state="fp32",
                                         slot_in=[1], slot_out=[2], P=2)
    inp["g"] = (inp["g"] * 5.0).clamp(min=-4.5).contiguous()
    check(sh, inp, pool, si, so, what="strong decay", mode=MODES[mode])


# --------------------------------------------------- the gate's whole range --
# The decay gate is alpha = exp(g) for any g <= 0; g = -inf empties those
# state channels at that token ("SGLang之KV Cache内存池机制" section 8.5,
# h *= exp(g); the ReplaySSM exact-commit passage of xxmr.cn/news/181459).
# Token positions below: 37 is inside a 16-token sub-block, 64 a tile
# boundary, 80 a sub-block boundary.

def set_gates(inp, fn):
    g = f64(inp["g"]).astype(np.float32)
    fn(g)
    inp["g"] = torch.from_numpy(g).to(inp["g"].device)


def gate_pattern(g, pattern, kda, lens):
    cu = synth.cu_seqlens(lens)
    a, b = cu[0], cu[1]          # the first sequence takes the pattern
    if pattern == "minus30":
        g[a:b] = -30.0
    elif pattern == "alternating":  # -30 / 0 per key channel (KDA), per token (GDN)
        if kda:
            g[a:b, :, 0::2] = -30.0
            g[a:b, :, 1::2] = 0.0
        else:
            g[a:b:2] = -30.0
            g[a + 1:b:2] = 0.0
    elif pattern == "resets":
        for t in (37, 64, 80):
            g[a + t] = -np.inf
        if kda:
            g[a + 100, :, ::3] = -np.inf  # a reset of some key channels only
        g[cu[2] + 5] = -np.inf        # and one inside the third sequence
    else:
        raise ValueError(pattern)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
@pytest.mark.parametrize("pattern", ["minus30", "alternating", "resets"])
def test_prefill_exact_over_the_gate_range(pattern, kda, mode, dev):
    """g = -30 per token, -30 / 0 alternating, and -inf resets (mid
    sub-block, at a tile boundary, at a sub-block boundary, on some channels
    only) match the oracle in both modes; the mild sequences packed after
    the first are unaffected."""
    lens = [150, 40, 70]
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3010, dev, kda=kda, io="fp32",
                                         state="fp32", slot_in=[1, -1, 2], slot_out=[3, 4, 5],
                                         P=5)
    set_gates(inp, lambda g: gate_pattern(g, pattern, kda, lens))
    print(f"[prefill gates] {pattern} kda={kda} mode={mode}", flush=True)
    check(sh, inp, pool, si, so, what=f"{pattern} kda={kda} {mode}", mode=MODES[mode])


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
def test_strong_decay_sequence_packed_beside_a_mild_one(kda, mode, dev):
    """Sequence A (10 tokens, g = -30, a -inf reset at its token 5) and
    sequence B (mild gates) share the first tile and its first 16-token
    sub-block; B, and A too, match the oracle.  A third sequence starts in
    the same tile after a -inf gate at its first token."""
    lens = [10, 30, 60, 20]
    sh, inp, pool, si, so = prefill_case(lens, 1, 1, 3011, dev, kda=kda, io="fp32",
                                         state="fp32", slot_in=[1, 2, -1, 3],
                                         slot_out=[4, 5, 6, 7], P=7)

    def pattern(g):
        g[0:10] = -30.0
        g[5] = -np.inf
        g[40] = -np.inf
    set_gates(inp, pattern)
    check(sh, inp, pool, si, so, what=f"packed strong/mild kda={kda}", mode=MODES[mode])


@pytest.mark.parametrize("mode", list(MODES))
def test_bf16_io_with_resets(mode, dev):
    """bf16 I/O with every tenth token a -inf reset of all channels."""
    lens = [200, 57]
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3012, dev, slot_in=[1, -1],
                                         slot_out=[2, 3], P=3)

    def pattern(g):
        g[::10] = -np.inf
    set_gates(inp, pattern)
    check(sh, inp, pool, si, so, what=f"bf16 resets {mode}", mode=MODES[mode])


def test_split_through_slots_equals_one_call(dev):
    """One sequence processed in three scheduler chunks (128 + 100 + 72
    tokens), each chunk's end state handed to the next through a pool slot,
    matches the single call and the oracle."""
    lens = [300]
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3005, dev, slot_in=[-1], slot_out=[1], P=3)
    pool2 = pool.clone()
    one = check(sh, inp, pool, si, so, what="one call")
    cuts = [0, 128, 228, 300]
    outs = []
    for c in range(3):
        a, b = cuts[c], cuts[c + 1]
        sub = {x: inp[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")}
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        csh = synth.PrefillShape(seqlens=(b - a,), Hqk=2, Hv=2, dk=D, dv=D)
        outs.append(run_gpu(csh, sub, pool2, np.array([-1 if c == 0 else 2], np.int32),
                            np.array([2], np.int32)))
    torch.cuda.synchronize()
    split = torch.cat(outs)
    assert_close_seqs(f64(split), f64(one), [0, 300], "bf16", "split vs one call outputs")
    assert_close_units(f64(pool2[2]), f64(pool[1]), 1, "fp32", "split vs one call state")


def test_packing_aligned_sequences_is_bit_exact(dev):
    lens = [128, 64, 192]
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3006, dev, slot_in=[1, 2, -1],
                                         slot_out=[4, 5, 6], P=9)
    pool_sep = pool.clone()
    packed = run_gpu(sh, inp, pool, si, so)
    cu = synth.cu_seqlens(lens)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sub = {x: inp[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")}
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        o = run_gpu(sh, sub, pool_sep, si[n:n + 1], so[n:n + 1])
        torch.cuda.synchronize()
        assert torch.equal(o, packed[a:b]), n
    assert torch.equal(pool, pool_sep)


def test_strided_qkv_views_of_conv_output(dev):
    """q, k, v given as token-strided views into one [T, C] tensor."""
    lens = [70, 30]
    Hqk = Hv = 2
    sh, inp, pool, si, so = prefill_case(lens, Hqk, Hv, 3007, dev, slot_in=[-1, 1],
                                         slot_out=[2, 3], P=3)
    T = sum(lens)
    y = torch.cat([inp["q"].reshape(T, -1), inp["k"].reshape(T, -1), inp["v"].reshape(T, -1)], 1)
    views = dict(inp, q=y[:, :Hqk * D].unflatten(1, (Hqk, D)),
                 k=y[:, Hqk * D:2 * Hqk * D].unflatten(1, (Hqk, D)),
                 v=y[:, 2 * Hqk * D:].unflatten(1, (Hv, D)))
    pool2 = pool.clone()
    o1 = run_gpu(sh, inp, pool, si, so)
    o2 = run_gpu(sh, views, pool2, si, so)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(pool, pool2)


def test_checked_mode_prefill_slot_rule(dev, monkeypatch):
    """LA_CHECK=1: a sequence may not read a row another sequence writes
    (their workgroups would race); repeated slot_in values (rows only read)
    and slot_in == slot_out of the same sequence are allowed and match the
    oracle."""
    monkeypatch.setenv("LA_CHECK", "1")
    sh, inp, pool, si, so = prefill_case([30, 50, 20], 1, 1, 3013, dev, slot_in=[1, 4, 1],
                                         slot_out=[2, 3, 1], P=5)
    # sequence 0 reads row 1, which sequence 2 writes (and 1 reads row 2 of 0)
    with pytest.raises(la.LAError, match="slot_out"):
        run_gpu(sh, inp, pool, np.array([1, 2, 5], np.int32), so)
    with pytest.raises(la.LAError, match="repeats"):
        run_gpu(sh, inp, pool, si, np.array([2, 3, 2], np.int32))
    # sequences 0 and 1 both read row 4; sequence 2 updates row 1 in place
    check(sh, inp, pool, np.array([4, 4, 1], np.int32), np.array([2, 3, 1], np.int32),
          what="checked slots")


def test_workspace_too_small_is_rejected(dev):
    sh, inp, pool, si, so = prefill_case([64], 1, 1, 3008, dev, P=2)
    with pytest.raises(la.LAError, match="workspace"):
        run_gpu(sh, inp, pool, si, so, workspace=torch.empty(1024, dtype=torch.uint8, device=dev))


# ---------------------------------------------------------------- sampled --

@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
def test_sampled_kda_prefill_long_sequence_in_scheduler_chunks(mode, dev):
    """KDA prefill at the serving shape: H=12, d=128, bf16 I/O, fp32 state; one
    13,600-token sequence in 6,144 / 6,144 / 1,312-token scheduler chunks, the
    end-of-chunk state written to a pool slot each chunk.  Heads 0 and 7 are
    checked against the oracle."""
    H = 12
    sh = synth.PrefillShape(seqlens=(13600,), Hqk=H, Hv=H, dk=D, dv=D)
    inp = synth.prefill_inputs(sh, 1005, dev)
    pool = torch.zeros((4, H, D, D), dtype=torch.float32, device=dev)
    heads = [0, 7]
    o_ref, p_ref = run_oracle(sh, inp, pool, np.array([-1], np.int32), np.array([1], np.int32),
                              heads)
    cuts = [0, 6144, 12288, 13600]
    outs = []
    for c in range(3):
        a, b = cuts[c], cuts[c + 1]
        sub = {x: inp[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")}
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        csh = synth.PrefillShape(seqlens=(b - a,), Hqk=H, Hv=H, dk=D, dv=D)
        # chunk c resumes from the slot chunk c - 1 wrote (slot c) and writes slot c + 1
        slot_in = np.array([-1 if c == 0 else c], np.int32)
        outs.append(run_gpu(csh, sub, pool, slot_in, np.array([c + 1], np.int32),
                            mode=MODES[mode]))
    torch.cuda.synchronize()
    out = f64(torch.cat(outs))[:, heads]
    assert_close_seqs(out, o_ref, [0, 13600], "bf16", "13600-token outputs (sampled heads)")
    assert_close_units(f64(pool[3])[heads], p_ref[1], 1, "fp32", "end state (sampled heads)")


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
def test_sampled_gdn_prefill_long_sequence_in_scheduler_chunks(mode, dev):
    """GDN prefill with 16 q/k heads shared by 32 value heads, bf16 I/O, fp32
    state: one 13,600-token sequence in 6,144 / 6,144 / 1,312-token scheduler
    chunks through pool slots (one sequence: the chain's 16-row form; in
    bf16x3 mode it reads the q rows and kernel 1's per-token scale).  Value
    heads 4 and 5 (both reading q/k head 2) and 30 are checked against the
    oracle."""
    Hqk, Hv = 16, 32
    sh = synth.PrefillShape(seqlens=(13600,), Hqk=Hqk, Hv=Hv, dk=D, dv=D, kda=False)
    inp = synth.prefill_inputs(sh, 1009, dev)
    pool = torch.zeros((4, Hv, D, D), dtype=torch.float32, device=dev)
    heads = [4, 5, 30]
    o_ref, p_ref = run_oracle(sh, inp, pool, np.array([-1], np.int32), np.array([1], np.int32),
                              heads)
    print(f"[prefill parity] gdn 16/32 heads 13600 tokens in 3 chunks mode={mode}", flush=True)
    cuts = [0, 6144, 12288, 13600]
    outs = []
    for c in range(3):
        a, b = cuts[c], cuts[c + 1]
        sub = {x: inp[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")}
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        csh = synth.PrefillShape(seqlens=(b - a,), Hqk=Hqk, Hv=Hv, dk=D, dv=D, kda=False)
        slot_in = np.array([-1 if c == 0 else c], np.int32)
        outs.append(run_gpu(csh, sub, pool, slot_in, np.array([c + 1], np.int32),
                            mode=MODES[mode]))
    torch.cuda.synchronize()
    split = mode == "bf16x3"
    out = f64(torch.cat(outs))[:, heads]
    assert_close_seqs(out, o_ref, [0, 13600], "bf16", "gdn 13600-token outputs (sampled heads)",
                      etol=elem_tol("bf16", split))
    assert_close_units(f64(pool[3])[heads], p_ref[1], 1, "fp32", "gdn end state (sampled heads)",
                       etol=elem_tol("fp32", split))


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
def test_sampled_kda_prefill_eight_packed_sequences(mode, dev):
    """Eight 4,096-token sequences packed into one varlen call (H=12), fresh
    states to eight distinct slots; heads 3 and 11 checked."""
    H = 12
    sh = synth.PrefillShape(seqlens=(4096,) * 8, Hqk=H, Hv=H, dk=D, dv=D)
    inp = synth.prefill_inputs(sh, 1006, dev)
    pool = torch.zeros((9, H, D, D), dtype=torch.float32, device=dev)
    si = np.full(8, -1, np.int32)
    so = np.arange(1, 9, dtype=np.int32)
    heads = [3, 11]
    o_ref, p_ref = run_oracle(sh, inp, pool, si, so, heads)
    out = run_gpu(sh, inp, pool, si, so, mode=MODES[mode])
    torch.cuda.synchronize()
    assert_close_seqs(f64(out)[:, heads], o_ref, synth.cu_seqlens(sh.seqlens), "bf16",
                      "packed outputs (sampled heads)")
    assert_close_units(f64(pool)[1:, heads], p_ref[1:], 2, "fp32", "packed end states")


@pytest.mark.parametrize("mode", ["fp32", "bf16x3"])
def test_sampled_gdn_prefill_gqa_eight_packed_sequences(mode, dev):
    """GDN prefill at its benchmarked shape: 16 q/k heads shared by 32 value
    heads, eight 4,096-token sequences packed into one call, bf16 I/O, fp32
    states.  Value heads 10 and 11 (both reading q/k head 5) and 31 are
    checked against the oracle."""
    sh = synth.PrefillShape(seqlens=(4096,) * 8, Hqk=16, Hv=32, dk=D, dv=D, kda=False)
    inp = synth.prefill_inputs(sh, 1007, dev)
    pool = torch.zeros((9, 32, D, D), dtype=torch.float32, device=dev)
    si = np.full(8, -1, np.int32)
    so = np.arange(1, 9, dtype=np.int32)
    heads = [10, 11, 31]
    o_ref, p_ref = run_oracle(sh, inp, pool, si, so, heads)
    print(f"[prefill parity] gdn 16/32 heads 8x4096 mode={mode}", flush=True)
    out = run_gpu(sh, inp, pool, si, so, mode=MODES[mode])
    torch.cuda.synchronize()
    assert_close_seqs(f64(out)[:, heads], o_ref, synth.cu_seqlens(sh.seqlens), "bf16",
                      "gdn packed outputs (sampled heads)")
    assert_close_units(f64(pool)[1:, heads], p_ref[1:], 2, "fp32", "gdn packed end states")


# ------------------------------------------------------------ short conv ---

@pytest.mark.parametrize("C", [8, 36, 4608])  # 36: the scalar path (C not a multiple of 8)
@pytest.mark.parametrize("io,cdt", [("bf16", "bf16"), ("fp32", "fp32"), ("fp32", "bf16"),
                                    ("bf16", "fp32")])
def test_shortconv_prefill_matches_oracle(io, cdt, C, dev):
    # sequences shorter than the window, an empty one, and sequences that
    # start inside and run across the 16-token runs of the vector path
    lens = [1, 2, 3, 40, 0, 9, 17, 33]
    N = len(lens)
    T = sum(lens)
    seed = 3100
    x = synth.to_torch(synth.normal(seed, 0, (T, C)), io, dev)
    w = synth.to_torch(0.5 * synth.normal(seed, 1, (C, 4)), "fp32", dev)
    P = 10
    pool = synth.to_torch(synth.normal(seed, 2, (P + 1, 3, C)), cdt, dev)
    si = np.array([4, -1, 5, 6, 7, -1, 3, 10], np.int32)
    so = np.array([4, 1, 2, 6, 8, 9, 3, 10], np.int32)   # four in place
    cu = synth.cu_seqlens(lens)
    y_ref, pool_ref = oracle.shortconv_prefill(f64(x), cu, si, so, f64(w), None, f64(pool),
                                               conv_dtype=cdt, io_dtype=io)
    y = la.shortconv_prefill(x, torch.from_numpy(cu).to(dev), torch.from_numpy(si).to(dev),
                             torch.from_numpy(so).to(dev), w, pool)
    torch.cuda.synchronize()
    assert_close_units(f64(y), y_ref, 1, io, "conv outputs")
    assert np.array_equal(f64(pool), pool_ref), "conv history must match bit for bit"


@pytest.mark.parametrize("C", [36, 4608])
def test_shortconv_prefill_skips_out_of_range_slots(C, dev):
    """A sequence whose slot is out of range gets zero outputs and touches no
    pool row; the other sequences are unaffected."""
    lens = [5, 20, 7]
    T = sum(lens)
    x = synth.to_torch(synth.normal(3102, 0, (T, C)), "bf16", dev)
    w = synth.to_torch(0.5 * synth.normal(3102, 1, (C, 4)), "fp32", dev)
    P = 4
    pool = synth.to_torch(synth.normal(3102, 2, (P + 1, 3, C)), "bf16", dev)
    before = pool.clone()
    cu = synth.cu_seqlens(lens)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    y = la.shortconv_prefill(x, torch.from_numpy(cu).to(dev), i32([1, 2, P + 1]),
                             i32([1, P + 7, 3]), w, pool)
    torch.cuda.synchronize()
    y_ref, pool_ref = oracle.shortconv_prefill(f64(x)[:5], [0, 5], [1], [1], f64(w), None,
                                               f64(before), conv_dtype="bf16", io_dtype="bf16")
    assert_close_units(f64(y)[:5], y_ref, 1, "bf16", "valid sequence")
    assert torch.count_nonzero(y[5:]) == 0
    assert np.array_equal(f64(pool)[1], pool_ref[1])
    assert torch.equal(pool[2:], before[2:]) and torch.equal(pool[0], before[0])


def test_shortconv_prefill_then_decode_continues_history(dev):
    """Prefill conv of a 50-token sequence, then one decode token through the
    standalone conv, equals the conv of the 51-token sequence."""
    C, L = 4608, 50
    x = synth.to_torch(synth.normal(3101, 0, (L + 1, C)), "bf16", dev)
    w = synth.to_torch(0.5 * synth.normal(3101, 1, (C, 4)), "fp32", dev)
    pool = torch.zeros((3, 3, C), dtype=torch.bfloat16, device=dev)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    y_all = la.shortconv_prefill(x, i32([0, L + 1]), i32([-1]), i32([2]), w, pool)
    la.shortconv_prefill(x[:L].contiguous(), i32([0, L]), i32([-1]), i32([1]), w, pool)
    y_last = la.shortconv_update(x[L:].contiguous(), w, pool, i32([1]))
    torch.cuda.synchronize()
    assert torch.equal(y_last[0], y_all[L])
    assert torch.equal(pool[1], pool[2])


@pytest.mark.parametrize("lens", [[40, 100, 7], [23 + 9 * n for n in range(30)]],
                         ids=["3seq", "30seq"])
def test_graph_replay_matches_eager(lens, dev):
    """Chunked prefill (bf16x3) captured in a HIP graph and replayed several
    times, each replay continuing the states in place, with eager work and
    synchronisations between replays: bit-identical to eager calls at every
    replay.  Thirty sequences x 2 heads take the chain's 64-row form (its
    masked buffer stores and register-held state)."""
    N = len(lens)
    slots = list(range(1, N + 1))
    sh, inp, pool, si, so = prefill_case(lens, 2, 2, 3400, dev, slot_in=slots, slot_out=slots,
                                         P=N + 1)
    si_t, so_t = torch.from_numpy(si).to(dev), torch.from_numpy(so).to(dev)
    pool_b = pool.clone()
    mode = la.LA_PREFILL_BF16X3
    ws = torch.empty(la.prefill_workspace_bytes(len(lens), sum(lens), 2, 2, D, D, mode),
                     dtype=torch.uint8, device=dev)
    out_b = torch.empty((sum(lens), 2, D), dtype=inp["q"].dtype, device=dev)

    def call(p, out=None, workspace=None):
        return la.kda_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      inp["cu_seqlens"], si_t, so_t, p, mode=mode, out=out,
                                      workspace=workspace)

    call(pool_b, out_b, ws)   # warm-up outside capture
    call(pool)                # keep the two pools in step
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(pool_b, out_b, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        out_a = call(pool)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), rep
        assert torch.equal(pool, pool_b), rep
