"""GPU parity of the fused decode step and the standalone short conv against
the fp64 oracle, through the C ABI.

Bars: conv-state contents and untouched pool rows bit-exact; outputs and
states within the relative-L2 tolerance of their storage dtype (1e-4 fp32,
2e-2 bf16) per (request, head); alpha = 1, beta = 0 leaves the state
bit-identical; permuting the batch with its slots is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_amd import binding as la
from linear_attention_recurrent_amd import synth
from parity_util import TOL, assert_close_units, dtype_name, f64

pytestmark = pytest.mark.gpu


def run_decode(sh, inp, **kw):
    fn = la.kda_decode_step if sh.kda else la.gdn_decode_step
    return fn(inp["x"], inp["g"], inp["beta"], inp["slots"], inp["ssm_pool"], Hqk=sh.Hqk,
              conv_w=inp["w"], conv_pool=inp["conv_pool"], **kw)


def oracle_decode(sh, inp, conv=True, **kw):
    return oracle.decode(f64(inp["x"]), f64(inp["w"]) if conv else None, None,
                         f64(inp["conv_pool"]), f64(inp["g"]), f64(inp["beta"]),
                         inp["slots"].cpu().numpy(), f64(inp["ssm_pool"]), Hqk=sh.Hqk, Hv=sh.Hv,
                         dk=sh.dk, dv=sh.dv, kda=sh.kda, conv_dtype=sh.conv,
                         state_dtype=sh.state, io_dtype=sh.io, **kw)


def check_step(sh, inp, dev, conv=True):
    """One decode step on the GPU vs the oracle; returns the GPU tensors."""
    before = {k: v.clone() for k, v in inp.items()}
    o_ref, cp_ref, sp_ref = oracle_decode(sh, before, conv)
    if not conv:
        inp = dict(inp, w=None)
    out = run_decode(sh, inp)
    torch.cuda.synchronize()
    slots = before["slots"].cpu().numpy()
    assert_close_units(f64(out), o_ref, 2, sh.io, "output")
    sp = f64(inp["ssm_pool"])
    assert_close_units(sp[slots], sp_ref[slots], 2, sh.state, "state")
    untouched = np.setdiff1d(np.arange(sh.P + 1), slots)
    assert np.array_equal(sp[untouched], f64(before["ssm_pool"])[untouched])
    cp = f64(inp["conv_pool"])
    assert np.array_equal(cp, cp_ref), "conv state must match bit for bit"
    return out


CASES = [
    # (name, shape)
    ("kda_bf16_d128", synth.DecodeShape(B=6, Hqk=3, Hv=3, dk=128, dv=128, P=9)),
    ("kda_fp32_d128", synth.DecodeShape(B=5, Hqk=2, Hv=2, dk=128, dv=128, P=8, io="fp32",
                                        state="fp32", conv="fp32")),
    ("gdn_fp32_gqa2_d128", synth.DecodeShape(B=4, Hqk=2, Hv=4, dk=128, dv=128, P=6, kda=False,
                                             io="fp32", state="fp32", conv="fp32")),
    ("gdn_bf16_gqa4_d64", synth.DecodeShape(B=3, Hqk=1, Hv=4, dk=64, dv=64, P=5, kda=False)),
    ("kda_mixed_d64", synth.DecodeShape(B=3, Hqk=2, Hv=2, dk=64, dv=64, P=4, io="bf16",
                                        state="fp32", conv="fp32")),
    ("kda_mixed2_d32", synth.DecodeShape(B=7, Hqk=2, Hv=4, dk=32, dv=32, P=9, io="fp32",
                                         state="bf16", conv="bf16")),
    ("gdn_bf16_d16", synth.DecodeShape(B=3, Hqk=2, Hv=2, dk=16, dv=16, P=4, kda=False)),
    ("kda_fp32_d16", synth.DecodeShape(B=2, Hqk=1, Hv=2, dk=16, dv=16, P=3, io="fp32",
                                       state="fp32", conv="bf16")),
]


@pytest.mark.parametrize("name,sh", CASES, ids=[c[0] for c in CASES])
def test_decode_step_matches_oracle(name, sh, dev):
    print(f"[decode parity] {name} {sh}", flush=True)
    inp = synth.decode_inputs(sh, 1100 + CASES.index((name, sh)), dev)
    check_step(sh, inp, dev)


@pytest.mark.parametrize("kda", [True, False], ids=["kda", "gdn"])
def test_decode_full_reset_gate(kda, dev):
    """g = -inf empties the state at this step (exp(-inf) = 0): for KDA on
    every other key channel of request 0 and all channels of request 2, for
    GDN on the heads of requests 0 and 2."""
    sh = synth.DecodeShape(B=4, Hqk=2, Hv=2, dk=128, dv=128, P=6, kda=kda, io="fp32",
                           state="fp32", conv="fp32")
    inp = synth.decode_inputs(sh, 1190 + kda, dev)
    g = inp["g"].cpu().clone()
    if kda:
        g[0, :, 0::2] = float("-inf")
    else:
        g[0] = float("-inf")
    g[2] = float("-inf")
    inp["g"] = g.to(dev)
    out = check_step(sh, inp, dev)
    assert torch.isfinite(out).all()


def test_decode_without_conv(dev):
    sh = synth.DecodeShape(B=4, Hqk=2, Hv=2, dk=128, dv=128, P=5, io="fp32", state="fp32",
                           conv="fp32")
    inp = synth.decode_inputs(sh, 1200, dev)
    check_step(sh, inp, dev, conv=False)


def test_tiny_gdn_layer_64_sequential_steps(dev):
    """Tiny GDN-style layer, fp32: batch 1, H=2, d=16, T=64 sequential tokens,
    conv weights 0.5 randn, zero initial state and conv state."""
    sh = synth.DecodeShape(B=1, Hqk=2, Hv=2, dk=16, dv=16, P=1, kda=False, io="fp32",
                           state="fp32", conv="fp32")
    seed = 1000
    T = 64
    C = sh.C
    xs = synth.normal(seed, synth.S_X, (T, C))
    w = synth.to_torch(0.5 * synth.normal(seed, synth.S_W, (C, 4)), "fp32", dev)
    g = synth.log_decay(seed, synth.S_G, (T, 2))
    beta = synth.beta_gate(seed, synth.S_BETA, (T, 2))
    conv_pool = torch.zeros((2, 3, C), dtype=torch.float32, device=dev)
    ssm_pool = torch.zeros((2, 2, 16, 16), dtype=torch.float32, device=dev)
    slots = torch.tensor([1], dtype=torch.int32, device=dev)
    cp, sp = np.zeros((2, 3, C)), np.zeros((2, 2, 16, 16))
    for t in range(T):
        x = synth.to_torch(xs[t:t + 1], "fp32", dev)
        gt = torch.from_numpy(g[t:t + 1]).to(dev)
        bt = torch.from_numpy(beta[t:t + 1]).to(dev)
        out = la.gdn_decode_step(x, gt, bt, slots, ssm_pool, Hqk=2, conv_w=w, conv_pool=conv_pool)
        o_ref, cp, sp = oracle.decode(f64(x), f64(w), None, cp, g[t:t + 1], beta[t:t + 1], [1], sp,
                                      Hqk=2, Hv=2, dk=16, dv=16, kda=False)
        assert_close_units(f64(out), o_ref, 2, "fp32", f"output step {t}")
    torch.cuda.synchronize()
    assert_close_units(f64(ssm_pool)[1], sp[1], 1, "fp32", "final state")
    assert np.array_equal(f64(conv_pool), cp)


def test_kda_single_layer_decode_full_shape(dev):
    """KDA decode step at the single-layer serving shape: 64 requests, H=12,
    d=128, bf16 state in an 80-slot pool (81 rows), random distinct slots,
    bf16 conv state; three consecutive steps."""
    sh = synth.DecodeShape(B=64, Hqk=12, Hv=12, dk=128, dv=128, P=80)
    inp = synth.decode_inputs(sh, 1001, dev)
    for step in range(3):
        print(f"[decode parity] full KDA layer step {step}", flush=True)
        check_step(sh, inp, dev)
        # next token: fresh x, g, beta (same slots, evolved pools)
        nxt = synth.decode_inputs(sh, 2000 + step, dev)
        for k in ("x", "g", "beta"):
            inp[k] = nxt[k]


def test_gdn_fp32_gqa_full_batch(dev):
    """GDN decode, fp32 state, 256 requests, 16 q/k heads shared by 32 value
    heads, d=128, one layer of the 48-layer stack."""
    sh = synth.DecodeShape(B=256, Hqk=16, Hv=32, dk=128, dv=128, P=256, kda=False, io="fp32",
                           state="fp32", conv="fp32")
    inp = synth.decode_inputs(sh, 1003, dev)
    check_step(sh, inp, dev)


@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_alpha_one_beta_zero_is_bit_exact(state, dev):
    sh = synth.DecodeShape(B=8, Hqk=4, Hv=4, dk=128, dv=128, P=10, state=state, conv=state)
    inp = synth.decode_inputs(sh, 1300, dev)
    inp["g"].zero_()
    inp["beta"].zero_()
    before = inp["ssm_pool"].clone()
    run_decode(sh, inp)
    torch.cuda.synchronize()
    assert torch.equal(inp["ssm_pool"], before)


def test_batch_permutation_is_bit_exact(dev):
    sh = synth.DecodeShape(B=16, Hqk=4, Hv=8, dk=128, dv=128, P=20, kda=False)
    a = synth.decode_inputs(sh, 1400, dev)
    b = {k: v.clone() for k, v in a.items()}
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(3)).to(dev)
    for k in ("x", "g", "beta", "slots"):
        b[k] = b[k][perm].contiguous()
    oa = run_decode(sh, a)
    ob = run_decode(sh, b)
    torch.cuda.synchronize()
    assert torch.equal(oa[perm], ob)
    assert torch.equal(a["ssm_pool"], b["ssm_pool"])
    assert torch.equal(a["conv_pool"], b["conv_pool"])


def test_out_of_range_slot_is_skipped(dev):
    sh = synth.DecodeShape(B=4, Hqk=2, Hv=2, dk=64, dv=64, P=6)
    inp = synth.decode_inputs(sh, 1500, dev)
    inp["slots"][2] = 99
    before_s, before_c = inp["ssm_pool"].clone(), inp["conv_pool"].clone()
    out = run_decode(sh, inp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[2]) == 0
    touched = inp["slots"][[0, 1, 3]].long()
    keep = torch.ones(sh.P + 1, dtype=torch.bool, device=dev)
    keep[touched] = False
    assert torch.equal(inp["ssm_pool"][keep], before_s[keep])
    assert torch.equal(inp["conv_pool"][keep], before_c[keep])


def test_checked_mode_rejects_duplicate_slots(dev, monkeypatch):
    sh = synth.DecodeShape(B=4, Hqk=2, Hv=2, dk=64, dv=64, P=6)
    inp = synth.decode_inputs(sh, 1501, dev)
    inp["slots"][3] = inp["slots"][1]
    monkeypatch.setenv("LA_CHECK", "1")
    with pytest.raises(la.LAError, match="repeats a slot"):
        run_decode(sh, inp)
    inp["slots"][3] = 7
    with pytest.raises(la.LAError, match="outside"):
        run_decode(sh, inp)


def test_padding_slot_zero_shared_by_several_entries(dev):
    sh = synth.DecodeShape(B=6, Hqk=2, Hv=2, dk=128, dv=128, P=8)
    inp = synth.decode_inputs(sh, 1502, dev)
    inp["slots"][1] = 0
    inp["slots"][4] = 0
    before = {k: v.clone() for k, v in inp.items()}
    out = run_decode(sh, inp)
    torch.cuda.synchronize()
    o_ref, _, sp_ref = oracle_decode(sh, before)
    real = [0, 2, 3, 5]
    assert_close_units(f64(out)[real], o_ref[real], 2, "bf16", "non-padded outputs")
    s = before["slots"].cpu().numpy()[real]
    assert_close_units(f64(inp["ssm_pool"])[s], sp_ref[s], 2, "bf16", "non-padded states")


@pytest.mark.parametrize("xdt,cdt", [("bf16", "bf16"), ("fp32", "fp32"), ("fp32", "bf16")])
def test_shortconv_update_matches_oracle(xdt, cdt, dev):
    B, C, P = 33, 4608 + 64, 40
    seed = 1600
    x = synth.to_torch(synth.normal(seed, 0, (B, C)), xdt, dev)
    w = synth.to_torch(0.5 * synth.normal(seed, 1, (C, 4)), "fp32", dev)
    bias = synth.to_torch(synth.normal(seed, 2, (C,)), "fp32", dev)
    pool = synth.to_torch(synth.normal(seed, 3, (P + 1, 3, C)), cdt, dev)
    slots = torch.from_numpy(synth.slot_permutation(seed, 4, P)[:B].copy()).to(dev)
    y_ref, pool_ref = oracle.shortconv_step(f64(x), f64(w), f64(bias), f64(pool),
                                            slots.cpu().numpy(), conv_dtype=cdt)
    y = la.shortconv_update(x, w, pool, slots, bias=bias)
    torch.cuda.synchronize()
    assert_close_units(f64(y), oracle.round_to(y_ref, xdt), 1, xdt, "conv output")
    assert np.array_equal(f64(pool), pool_ref)


def test_fused_prologue_equals_standalone_conv(dev):
    """The fused decode's conv-state update equals the standalone call's."""
    sh = synth.DecodeShape(B=8, Hqk=4, Hv=8, dk=128, dv=128, P=12, kda=False)
    a = synth.decode_inputs(sh, 1700, dev)
    pool2 = a["conv_pool"].clone()
    run_decode(sh, a)
    la.shortconv_update(a["x"], a["w"], pool2, a["slots"])
    torch.cuda.synchronize()
    assert torch.equal(a["conv_pool"], pool2)


def _sampled_full_shape(sh, seed, dev, n_sample):
    inp = synth.decode_inputs(sh, seed, dev)
    pick = np.sort(np.random.default_rng(seed).choice(sh.B, n_sample, replace=False))
    slots = inp["slots"].cpu().numpy()
    sub = dict(
        x=f64(inp["x"][pick]), w=f64(inp["w"]), g=f64(inp["g"][pick]),
        beta=f64(inp["beta"][pick]),
        conv_pool=np.concatenate([np.zeros((1, 3, sh.C)), f64(inp["conv_pool"][slots[pick]])]),
        ssm_pool=np.concatenate([np.zeros((1, sh.Hv, sh.dv, sh.dk)),
                                 f64(inp["ssm_pool"][slots[pick]])]))
    out = run_decode(sh, inp)
    torch.cuda.synchronize()
    o_ref, cp_ref, sp_ref = oracle.decode(
        sub["x"], sub["w"], None, sub["conv_pool"], sub["g"], sub["beta"],
        np.arange(1, n_sample + 1), sub["ssm_pool"], Hqk=sh.Hqk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv,
        kda=sh.kda, conv_dtype=sh.conv, state_dtype=sh.state, io_dtype=sh.io)
    assert_close_units(f64(out[pick]), o_ref, 2, sh.io, "sampled outputs")
    assert_close_units(f64(inp["ssm_pool"][slots[pick]]), sp_ref[1:], 2, sh.state,
                       "sampled states")
    assert np.array_equal(f64(inp["conv_pool"][slots[pick]]), cp_ref[1:])


def test_sampled_parity_kda_96_heads_128_requests(dev):
    """One layer of the 69-layer KDA stack at its full per-layer shape
    (H=96, d=128, 128 requests, bf16 state, 129-row pool): 6 sampled requests
    x 96 heads checked against the oracle."""
    sh = synth.DecodeShape(B=128, Hqk=96, Hv=96, dk=128, dv=128, P=128)
    _sampled_full_shape(sh, 1002, dev, 6)


def test_sampled_parity_gdn_fp32_256_requests(dev):
    sh = synth.DecodeShape(B=256, Hqk=16, Hv=32, dk=128, dv=128, P=256, kda=False, io="fp32",
                           state="fp32", conv="fp32")
    _sampled_full_shape(sh, 1004, dev, 12)


def test_graph_replay_matches_eager(dev):
    """Decode captured in a HIP graph and replayed several times, with eager
    work and synchronisations between replays, equals eager calls bit for bit
    at every replay."""
    sh = synth.DecodeShape(B=16, Hqk=4, Hv=4, dk=128, dv=128, P=20)
    a = synth.decode_inputs(sh, 1800, dev)
    b = {k: v.clone() for k, v in a.items()}
    out_b = torch.empty((sh.B, sh.Hv, sh.dv), dtype=torch.bfloat16, device=dev)
    run_decode(sh, b, out=out_b)          # warm-up call outside capture
    run_decode(sh, a)                     # keep a and b in step
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_decode(sh, b, out=out_b)
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        out_a = run_decode(sh, a)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), rep
        assert torch.equal(a["ssm_pool"], b["ssm_pool"]), rep
        assert torch.equal(a["conv_pool"], b["conv_pool"]), rep
