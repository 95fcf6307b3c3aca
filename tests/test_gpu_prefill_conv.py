"""GPU parity of the chunked prefill with the short conv fused into its loads
(kda_prefill_conv / gdn_prefill_conv) against the fp64 oracle, through the
C ABI.

The oracle runs the two steps the fused call merges: the varlen short conv
(its activations left unrounded, since the fused path keeps them in fp32)
and the token-by-token prefill on the conv output split into q | k | v.

Bars: conv-pool contents bit-exact; outputs and final states within the
relative L2 tolerance of their storage dtype per (token or slot, head); with
fp32 I/O the fused call equals the standalone conv followed by the chunked
prefill bit for bit (same taps, same sum order, no rounding in between).
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
MODES = {"fp32": la.LA_PREFILL_FP32, "bf16x3": la.LA_PREFILL_BF16X3}


def conv_case(lens, Hqk, Hv, seed, dev, *, kda=True, io="bf16", state="fp32", cdt="bf16",
              slot_in, slot_out, P, bias=True):
    """Pre-conv projections x [T, C] (randn), conv taps 0.5 randn, bias 0.1
    randn, random conv and SSM pools; g and beta as the other prefill tests."""
    sh = synth.PrefillShape(seqlens=tuple(lens), Hqk=Hqk, Hv=Hv, dk=D, dv=D, kda=kda, io=io,
                            state=state)
    inp = synth.prefill_inputs(sh, seed, dev)
    T, C = sh.T, 2 * Hqk * D + Hv * D
    x = synth.to_torch(synth.normal(seed, 10, (T, C)), io, dev)
    w = synth.to_torch(0.5 * synth.normal(seed, 11, (C, 4)), "fp32", dev)
    b = synth.to_torch(0.1 * synth.normal(seed, 12, (C,)), "fp32", dev) if bias else None
    cpool = synth.to_torch(synth.normal(seed, 13, (P + 1, 3, C)), cdt, dev)
    spool = synth.normal_torch(seed, synth.S_SSM, (P + 1) * Hv * D * D, dev,
                               synth.TORCH_DTYPE[state]).view(P + 1, Hv, D, D)
    return dict(sh=sh, x=x, w=w, b=b, cpool=cpool, spool=spool, g=inp["g"], beta=inp["beta"],
                cu=inp["cu_seqlens"], si=np.array(slot_in, np.int32),
                so=np.array(slot_out, np.int32), cdt=cdt)


def run_fused(c, dev, **kw):
    fn = la.kda_prefill_conv if c["sh"].kda else la.gdn_prefill_conv
    return fn(c["x"], c["g"], c["beta"], c["cu"], torch.from_numpy(c["si"]).to(dev),
              torch.from_numpy(c["so"]).to(dev), c["spool"], Hqk=c["sh"].Hqk, conv_w=c["w"],
              conv_b=c["b"], conv_pool=c["cpool"], **kw)


def run_oracle(c, cpool, spool):
    sh = c["sh"]
    T, Hqk, Hv = sh.T, sh.Hqk, sh.Hv
    cu = c["cu"].cpu().numpy()
    y, cpool_ref = oracle.shortconv_prefill(f64(c["x"]), cu, c["si"], c["so"], f64(c["w"]),
                                            None if c["b"] is None else f64(c["b"]), f64(cpool),
                                            conv_dtype=c["cdt"], io_dtype="fp64")
    q = y[:, :Hqk * D].reshape(T, Hqk, D)
    k = y[:, Hqk * D:2 * Hqk * D].reshape(T, Hqk, D)
    v = y[:, 2 * Hqk * D:].reshape(T, Hv, D)
    o, spool_ref = oracle.prefill(q, k, v, f64(c["g"]), f64(c["beta"]), cu, c["si"], c["so"],
                                  f64(spool), kda=sh.kda, state_dtype=sh.state, io_dtype=sh.io)
    return o, cpool_ref, spool_ref


def check(c, dev, what, mode):
    cbefore, sbefore = c["cpool"].clone(), c["spool"].clone()
    o_ref, cpool_ref, spool_ref = run_oracle(c, cbefore, sbefore)
    print(f"[fused conv prefill] {what}", flush=True)
    out = run_fused(c, dev, mode=MODES[mode])
    torch.cuda.synchronize()
    sh, so = c["sh"], c["so"]
    split = MODES[mode] == la.LA_PREFILL_BF16X3  # split products: the derived element bar
    assert_close_seqs(f64(out), o_ref, c["cu"].cpu().numpy(), sh.io, f"{what} outputs",
                      etol=elem_tol(sh.io, split))
    assert_close_units(f64(c["spool"])[so], spool_ref[so], 2, sh.state, f"{what} final states",
                       etol=elem_tol(sh.state, split))
    assert np.array_equal(f64(c["cpool"]), cpool_ref), f"{what}: conv pool must match bit for bit"
    untouched = np.setdiff1d(np.arange(c["spool"].shape[0]), so)
    assert torch.equal(c["spool"][untouched], sbefore[untouched])
    return out


# sequences shorter than the conv window, an empty one, one that fills a
# tile exactly and ones that cross tile boundaries, several inside one tile
LENS = [1, 2, 3, 70, 0, 130, 5, 64]
SI = [4, -1, 5, 6, 7, -1, 3, 10]
SO = [4, 1, 2, 6, 8, 9, 3, 10]  # four sequences in place


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("io,state,cdt", [("bf16", "fp32", "bf16"), ("fp32", "fp32", "fp32"),
                                          ("bf16", "bf16", "fp32")])
def test_kda_prefill_conv_matches_oracle(io, state, cdt, mode, dev):
    c = conv_case(LENS, 2, 2, 3200, dev, io=io, state=state, cdt=cdt, slot_in=SI, slot_out=SO,
                  P=10)
    check(c, dev, f"kda io={io} state={state} conv={cdt} mode={mode}", mode)


@pytest.mark.parametrize("mode", list(MODES))
def test_gdn_prefill_conv_gqa_matches_oracle(mode, dev):
    c = conv_case(LENS, 1, 2, 3201, dev, kda=False, io="bf16", state="fp32", cdt="bf16",
                  slot_in=SI, slot_out=SO, P=10, bias=False)
    check(c, dev, f"gdn gqa mode={mode}", mode)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
def test_prefill_conv_with_strong_decay_and_resets(kda, mode, dev):
    """The fused call over the gate's whole range: a first sequence at
    g = -30 with a -inf reset, packed in one sub-block with a mild one, and
    -inf resets at a tile boundary and a sub-block boundary of the third
    ("SGLang之KV Cache内存池机制" section 8.5, h *= exp(g))."""
    c = conv_case([10, 30, 100], 1, 1, 3203, dev, kda=kda, io="fp32", state="fp32", cdt="fp32",
                  slot_in=[1, -1, 2], slot_out=[3, 4, 5], P=5)
    g = f64(c["g"]).astype(np.float32)
    g[0:10] = -30.0
    g[5] = -np.inf
    g[64] = -np.inf
    g[80] = -np.inf
    c["g"] = torch.from_numpy(g).to(dev)
    check(c, dev, f"gate range kda={kda} mode={mode}", mode)


@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
def test_prefill_conv_items_across_tiles_four_value_heads_per_qk_head(kda, dev):
    """More (tile, head) items than the persistent grid has workgroups (40
    to 46 tiles x 8 value heads), so workgroups take a second item one grid
    stride on, in another tile, and fetch its conv window history again.  Four
    value heads share each of the two q/k heads."""
    rng = np.random.default_rng(3400 + kda)
    lens = [int(x) for x in rng.integers(1, 300, size=16)]
    N = len(lens)
    si = [n + 1 if n % 3 == 0 else -1 for n in range(N)]
    so = [N + 1 + n for n in range(N)]
    c = conv_case(lens, 2, 8, 3210 + kda, dev, kda=kda, slot_in=si, slot_out=so, P=2 * N + 1)
    check(c, dev, f"items across tiles kda={kda}", "bf16x3")


def test_kda_prefill_conv_gqa_matches_oracle(dev):
    c = conv_case([65, 40, 2], 2, 4, 3202, dev, slot_in=[1, -1, 4], slot_out=[2, 3, 4], P=4)
    check(c, dev, "kda gqa", "bf16x3")


@pytest.mark.parametrize("kda", [True, False])
def test_fused_equals_standalone_conv_then_prefill_fp32(kda, dev):
    """fp32 I/O: shortconv_prefill followed by the chunked prefill on views of
    its output gives the fused call's outputs and pools bit for bit."""
    Hqk, Hv = 2, 2
    c = conv_case(LENS, Hqk, Hv, 3203, dev, kda=kda, io="fp32", state="fp32", cdt="fp32",
                  slot_in=SI, slot_out=SO, P=10)
    cpool2, spool2 = c["cpool"].clone(), c["spool"].clone()
    si, so = torch.from_numpy(c["si"]).to(dev), torch.from_numpy(c["so"]).to(dev)
    out = run_fused(c, dev)
    y = la.shortconv_prefill(c["x"], c["cu"], si, so, c["w"], cpool2, bias=c["b"])
    T = c["sh"].T
    fn = la.kda_prefill_chunked if kda else la.gdn_prefill_chunked
    out2 = fn(y[:, :Hqk * D].unflatten(1, (Hqk, D)), y[:, Hqk * D:2 * Hqk * D].unflatten(1, (Hqk, D)),
              y[:, 2 * Hqk * D:].unflatten(1, (Hv, D)), c["g"], c["beta"], c["cu"], si, so, spool2)
    torch.cuda.synchronize()
    assert out.shape == (T, Hv, D)
    assert torch.equal(out, out2)
    assert torch.equal(c["cpool"], cpool2)
    assert torch.equal(c["spool"], spool2)


def test_prefill_conv_skips_out_of_range_slots(dev):
    """A sequence with an out-of-range slot gets zero outputs and touches
    neither pool; the others match the oracle run without it."""
    P = 4
    c = conv_case([20, 9, 33], 1, 1, 3204, dev, io="bf16", state="fp32", cdt="bf16",
                  slot_in=[1, 2, P + 3], slot_out=[1, P + 9, 3], P=P)
    cbefore, sbefore = c["cpool"].clone(), c["spool"].clone()
    out = run_fused(c, dev)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[20:]) == 0
    sub = dict(c, sh=synth.PrefillShape(seqlens=(20,), Hqk=1, Hv=1, dk=D, dv=D),
               x=c["x"][:20], g=c["g"][:20], beta=c["beta"][:20],
               cu=torch.tensor([0, 20], dtype=torch.int32), si=c["si"][:1], so=c["so"][:1])
    o_ref, cpool_ref, spool_ref = run_oracle(sub, cbefore, sbefore)
    assert_close_seqs(f64(out)[:20], o_ref, [0, 20], "bf16", "valid sequence")
    assert np.array_equal(f64(c["cpool"]), cpool_ref)
    assert_close_units(f64(c["spool"])[1:2], spool_ref[1:2], 2, "fp32", "valid sequence state")
    assert torch.equal(c["spool"][2:], sbefore[2:]) and torch.equal(c["spool"][0], sbefore[0])


def test_prefill_conv_then_decode_continues(dev):
    """A 90-token sequence through the fused prefill, then its 91st token
    through the fused decode, matches the oracle over all 91 tokens."""
    Hqk = Hv = 1
    L = 90
    c = conv_case([L + 1], Hqk, Hv, 3205, dev, io="bf16", state="fp32", cdt="bf16",
                  slot_in=[-1], slot_out=[1], P=2)
    o_all, _, spool_ref = run_oracle(c, c["cpool"].clone(), c["spool"].clone())
    head = dict(c, sh=synth.PrefillShape(seqlens=(L,), Hqk=1, Hv=1, dk=D, dv=D),
                x=c["x"][:L].contiguous(), g=c["g"][:L].contiguous(),
                beta=c["beta"][:L].contiguous(),
                cu=torch.tensor([0, L], dtype=torch.int32, device=dev))
    o_head = run_fused(head, dev)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    # clones: the API wants 16-byte aligned buffers, a one-row slice may not be
    o_last = la.kda_decode_step(c["x"][L:].clone(), c["g"][L:].clone(),
                                c["beta"][L:].clone(), i32([1]), c["spool"], Hqk=Hqk,
                                conv_w=c["w"], conv_b=c["b"], conv_pool=c["cpool"])
    torch.cuda.synchronize()
    out = torch.cat([o_head, o_last])
    assert_close_seqs(f64(out), o_all, [0, L + 1], "bf16", "prefill + decode outputs")
    assert_close_units(f64(c["spool"])[1:2], spool_ref[1:2], 2, "fp32", "state after decode")


@pytest.mark.parametrize("mode", list(MODES))
def test_sampled_kda_prefill_conv_serving_shape(mode, dev):
    """Serving shape (H=12, d=128, bf16 I/O and conv pool, fp32 state): two
    sequences of 3,000 and 1,100 tokens resuming from conv and SSM history;
    the oracle runs on heads 0 and 9 only (their q, k, v channels of x)."""
    H = 12
    lens = [3000, 1100]
    c = conv_case(lens, H, H, 3206, dev, slot_in=[1, 2], slot_out=[3, 2], P=3)
    heads = [0, 9]
    C = 3 * H * D
    ch = np.concatenate([np.arange(h * D, (h + 1) * D) + blk * H * D
                         for blk in range(3) for h in heads])
    cbefore, sbefore = c["cpool"].clone(), c["spool"].clone()
    out = run_fused(c, dev, mode=MODES[mode])
    torch.cuda.synchronize()
    chd = torch.from_numpy(ch).to(dev)
    sub = dict(c, sh=synth.PrefillShape(seqlens=tuple(lens), Hqk=2, Hv=2, dk=D, dv=D),
               x=c["x"][:, chd], w=c["w"][chd], b=c["b"][chd], g=c["g"][:, heads],
               beta=c["beta"][:, heads])
    o_ref, cpool_ref, spool_ref = run_oracle(sub, cbefore[:, :, chd], sbefore[:, heads])
    assert_close_seqs(f64(out)[:, heads], o_ref, synth.cu_seqlens(lens), "bf16",
                      "outputs (sampled heads)")
    assert_close_units(f64(c["spool"])[:, heads][[3, 2]], spool_ref[[3, 2]], 2, "fp32",
                       "end states (sampled heads)")
    assert np.array_equal(f64(c["cpool"])[:, :, ch], cpool_ref)
    assert C == c["x"].shape[1]


@pytest.mark.parametrize("fused", [False, True])
def test_all_sequences_empty_hands_states_over(fused, dev):
    """T = 0 with N = 3: no tokens, so each sequence's slot_out receives its
    initial state (zeros when slot_in < 0) and, fused, its conv history."""
    c = conv_case([0, 0, 0], 1, 1, 3207, dev, slot_in=[2, -1, 4], slot_out=[5, 6, 4], P=6)
    cbefore, sbefore = c["cpool"].clone(), c["spool"].clone()
    if fused:
        out = run_fused(c, dev)
    else:
        Hqk, Hv = 1, 1
        empty = torch.empty((0, Hqk, D), dtype=torch.bfloat16, device=dev)
        out = la.kda_prefill_chunked(empty, empty, torch.empty((0, Hv, D), dtype=torch.bfloat16,
                                                               device=dev),
                                     c["g"], c["beta"], c["cu"], torch.from_numpy(c["si"]).to(dev),
                                     torch.from_numpy(c["so"]).to(dev), c["spool"])
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert torch.equal(c["spool"][5], sbefore[2])
    assert torch.count_nonzero(c["spool"][6]) == 0
    assert torch.equal(c["spool"][4], sbefore[4])
    for r in (0, 1, 2, 3):
        assert torch.equal(c["spool"][r], sbefore[r])
    if fused:
        assert torch.equal(c["cpool"][5], cbefore[2])
        assert torch.count_nonzero(c["cpool"][6]) == 0
        assert torch.equal(c["cpool"][4], cbefore[4])


@pytest.mark.parametrize("fused", [False, True])
def test_many_short_sequences_share_tiles(fused, dev):
    """70 sequences of 1-3 tokens (seeded lengths), so a 64-token tile holds
    dozens of pieces and the per-token sequence lookup runs deep; every
    other one resumes from a pool slot."""
    rng = np.random.default_rng(3208)
    lens = [int(x) for x in rng.integers(1, 4, size=70)]
    N = len(lens)
    si = [n + 1 if n % 2 else -1 for n in range(N)]
    so = [N + 1 + n for n in range(N)]
    c = conv_case(lens, 1, 2, 3208, dev, kda=False, io="bf16", state="fp32", cdt="bf16",
                  slot_in=si, slot_out=so, P=2 * N + 1)
    if fused:
        check(c, dev, "70 short sequences, fused", "bf16x3")
        return
    # unfused: the oracle's conv output (rounded to bf16 as a conv call would
    # store it) is the prefill's input
    sh = c["sh"]
    T = sh.T
    y, _ = oracle.shortconv_prefill(f64(c["x"]), c["cu"].cpu().numpy(), c["si"], c["so"],
                                    f64(c["w"]), f64(c["b"]), f64(c["cpool"]),
                                    conv_dtype="bf16", io_dtype="bf16")
    yt = torch.from_numpy(y).to(torch.bfloat16).to(dev)
    q = yt[:, :D].reshape(T, 1, D)
    k = yt[:, D:2 * D].reshape(T, 1, D)
    v = yt[:, 2 * D:].reshape(T, 2, D).contiguous()
    sbefore = c["spool"].clone()
    o_ref, s_ref = oracle.prefill(f64(q), f64(k), f64(v), f64(c["g"]), f64(c["beta"]),
                                  c["cu"].cpu().numpy(), c["si"], c["so"], f64(sbefore),
                                  kda=False, state_dtype="fp32", io_dtype="bf16")
    out = la.gdn_prefill_chunked(q.contiguous(), k.contiguous(), v, c["g"], c["beta"], c["cu"],
                                 torch.from_numpy(c["si"]).to(dev),
                                 torch.from_numpy(c["so"]).to(dev), c["spool"],
                                 mode=la.LA_PREFILL_BF16X3)
    torch.cuda.synchronize()
    assert_close_seqs(f64(out), o_ref, c["cu"].cpu().numpy(), "bf16", "70 short sequences outputs")
    assert_close_units(f64(c["spool"])[c["so"]], s_ref[c["so"]], 2, "fp32", "end states")
