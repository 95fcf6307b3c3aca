"""The Python binding rejects, before any launch, the arguments whose dtype,
shape or device the C ABI cannot check itself (it sees raw pointers only):
a wrong one would make a kernel read past an allocation or misread indices
(int64 slots read as int32 words name the wrong pool rows).  CPU tensors
throughout: every call here ends in a ValueError or TypeError and no library
call is made; with every tensor right, the last check refuses CPU memory."""
import re

import pytest
import torch

from linear_attention_recurrent_amd import binding as la

B, Hqk, Hv, D = 4, 2, 4, 128
C = 2 * Hqk * D + Hv * D
P = 6
f32, bf16, i32 = torch.float32, torch.bfloat16, torch.int32


def decode_args(kda=True):
    return dict(x=torch.zeros(B, C, dtype=bf16),
                g=torch.zeros((B, Hv, D) if kda else (B, Hv), dtype=f32),
                beta=torch.zeros(B, Hv, dtype=f32), slots=torch.arange(1, B + 1, dtype=i32),
                ssm_pool=torch.zeros(P + 1, Hv, D, D, dtype=bf16),
                conv_w=torch.zeros(C, 4, dtype=f32),
                conv_pool=torch.zeros(P + 1, 3, C, dtype=bf16))


def call_decode(kda, a):
    fn = la.kda_decode_step if kda else la.gdn_decode_step
    return fn(a["x"], a["g"], a["beta"], a["slots"], a["ssm_pool"], Hqk=Hqk,
              conv_w=a["conv_w"], conv_pool=a["conv_pool"])


@pytest.mark.parametrize("kda", [True, False])
@pytest.mark.parametrize("field,bad,msg", [
    ("slots", torch.arange(1, B + 1, dtype=torch.int64), "slots: dtype"),
    ("slots", torch.arange(1, B, dtype=torch.int32), "slots: shape"),
    ("beta", torch.zeros(B, Hv, dtype=torch.bfloat16), "beta: dtype"),
    ("beta", torch.zeros(B, Hv - 1, dtype=torch.float32), "beta: shape"),
    ("g", torch.zeros(B, Hv, 64, dtype=torch.float32), "g: shape"),
    ("g", torch.zeros(B, Hv, D, dtype=torch.float64), "g: dtype"),
    ("conv_w", torch.zeros(C, 4, dtype=torch.bfloat16), "conv_w: dtype"),
    ("conv_w", torch.zeros(C, 3, dtype=torch.float32), "conv_w: shape"),
    ("x", torch.zeros(B, C, dtype=torch.float16), "x: dtype"),
    ("ssm_pool", torch.zeros(P + 1, Hv, D, D, dtype=torch.float16), "ssm_pool: dtype"),
])
def test_decode_rejects(kda, field, bad, msg):
    a = decode_args(kda)
    if field == "g" and not kda and bad.dim() == 3 and bad.dtype == torch.float32:
        bad = torch.zeros(B, Hv + 1, dtype=f32)  # GDN gate shape [B, Hv]
    a[field] = bad
    with pytest.raises((ValueError, TypeError), match=re.escape(msg)):
        call_decode(kda, a)


def test_decode_gdn_rejects_a_kda_shaped_gate():
    a = decode_args(kda=False)
    a["g"] = torch.zeros(B, Hv, D, dtype=f32)
    with pytest.raises(ValueError, match="g: shape"):
        call_decode(False, a)


@pytest.mark.parametrize("kda", [True, False])
def test_decode_refuses_host_memory_last(kda):
    with pytest.raises(ValueError, match="GPU"):
        call_decode(kda, decode_args(kda))


def prefill_args(kda=True, N=3, T=40):
    return dict(q=torch.zeros(T, Hqk, D, dtype=bf16), k=torch.zeros(T, Hqk, D, dtype=bf16),
                v=torch.zeros(T, Hv, D, dtype=bf16),
                g=torch.zeros((T, Hv, D) if kda else (T, Hv), dtype=f32),
                beta=torch.zeros(T, Hv, dtype=f32),
                cu_seqlens=torch.tensor([0, 10, 30, T], dtype=i32),
                slot_in=torch.full((N,), -1, dtype=i32),
                slot_out=torch.arange(1, N + 1, dtype=i32),
                ssm_pool=torch.zeros(P + 1, Hv, D, D, dtype=f32))


def call_prefill(kda, a):
    fn = la.kda_prefill_chunked if kda else la.gdn_prefill_chunked
    return fn(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu_seqlens"], a["slot_in"],
              a["slot_out"], a["ssm_pool"])


@pytest.mark.parametrize("kda", [True, False])
@pytest.mark.parametrize("field,bad,msg", [
    ("cu_seqlens", torch.tensor([0, 10, 30, 40], dtype=torch.int64), "cu_seqlens: dtype"),
    ("slot_in", torch.full((2,), -1, dtype=torch.int32), "slot_in: shape"),
    ("slot_out", torch.arange(1, 4, dtype=torch.int64), "slot_out: dtype"),
    ("beta", torch.zeros(39, Hv, dtype=torch.float32), "beta: shape"),
    ("v", torch.zeros(40, Hv, D, dtype=torch.float32), "v: dtype"),
    ("k", torch.zeros(40, Hqk + 1, D, dtype=torch.bfloat16), "k: expected"),
])
def test_prefill_rejects(kda, field, bad, msg):
    a = prefill_args(kda)
    a[field] = bad
    with pytest.raises((ValueError, TypeError), match=re.escape(msg)):
        call_prefill(kda, a)


@pytest.mark.parametrize("kda", [True, False])
def test_prefill_gate_shape(kda):
    a = prefill_args(kda)
    a["g"] = torch.zeros((40, Hv) if kda else (40, Hv, D), dtype=f32)  # the other variant's
    with pytest.raises(ValueError, match="g: shape"):
        call_prefill(kda, a)


def test_prefill_refuses_host_memory_last():
    with pytest.raises(ValueError, match="GPU"):
        call_prefill(True, prefill_args())


def test_prefill_conv_rejects_int64_slots():
    a = prefill_args()
    with pytest.raises(ValueError, match="slot_out"):
        la.kda_prefill_conv(torch.zeros(40, C, dtype=bf16), a["g"], a["beta"], a["cu_seqlens"],
                            a["slot_in"], a["slot_out"].to(torch.int64), a["ssm_pool"], Hqk=Hqk,
                            conv_w=torch.zeros(C, 4, dtype=f32),
                            conv_pool=torch.zeros(P + 1, 3, C, dtype=bf16))


def test_shortconv_rejects():
    x = torch.zeros(B, C, dtype=bf16)
    pool = torch.zeros(P + 1, 3, C, dtype=bf16)
    w = torch.zeros(C, 4, dtype=f32)
    with pytest.raises(ValueError, match="slots"):
        la.shortconv_update(x, w, pool, torch.arange(1, B + 1))          # int64
    with pytest.raises(ValueError, match="bias"):
        la.shortconv_update(x, w, pool, torch.arange(1, B + 1, dtype=i32),
                            bias=torch.zeros(C - 1, dtype=f32))
    with pytest.raises(ValueError, match="GPU"):
        la.shortconv_update(x, w, pool, torch.arange(1, B + 1, dtype=i32))
    cu = torch.tensor([0, 2, B], dtype=i32)
    with pytest.raises(ValueError, match="slot_in"):
        la.shortconv_prefill(x, cu, torch.tensor([-1], dtype=i32), torch.tensor([1, 2], dtype=i32),
                             w, pool)


def spec_args(kda=True, Dd=4, L=8):
    return dict(x=torch.zeros(B, Dd, C, dtype=bf16),
                g=torch.zeros((B, Dd, Hv, D) if kda else (B, Dd, Hv), dtype=f32),
                beta=torch.zeros(B, Dd, Hv, dtype=f32), slots=torch.arange(1, B + 1, dtype=i32),
                n_tok=torch.full((B,), Dd, dtype=i32),
                ssm_pool=torch.zeros(P + 1, Hv, D, D, dtype=bf16),
                ring=la.new_ring(P + 1, Hv, L, D, D, kda=kda, dtype=bf16, device="cpu"),
                ring_base=torch.zeros(B, dtype=i32))


@pytest.mark.parametrize("kda", [True, False])
def test_verify_commit_fold_reject(kda):
    a = spec_args(kda)
    fn = la.kda_verify if kda else la.gdn_verify
    call = lambda **o: fn(**{**{k: a[k] for k in ("x", "g", "beta", "slots", "n_tok",  # noqa
                                                    "ssm_pool", "ring", "ring_base")}, **o},
                          Hqk=Hqk)
    with pytest.raises(ValueError, match="n_tok"):
        call(n_tok=torch.full((B,), 4, dtype=torch.int64))
    with pytest.raises(ValueError, match="ring_base"):
        call(ring_base=torch.zeros(B - 1, dtype=i32))
    bad_ring = dict(a["ring"], beta=torch.zeros(P, Hv, 8, dtype=f32))  # one row short
    with pytest.raises(ValueError, match="ring"):
        call(ring=bad_ring)
    f32_ring = la.new_ring(P + 1, Hv, 8, D, D, kda=kda, dtype=f32, device="cpu")
    with pytest.raises(ValueError, match="ring"):                     # x is bf16
        call(ring=f32_ring)
    with pytest.raises(ValueError, match="GPU"):
        call()
    commit = la.kda_commit if kda else la.gdn_commit
    with pytest.raises(ValueError, match="accepted"):
        commit(torch.ones(B, dtype=torch.int64), a["slots"], a["ssm_pool"], a["ring"],
               a["ring_base"])
    with pytest.raises(ValueError, match="GPU"):
        commit(torch.ones(B, dtype=i32), a["slots"], a["ssm_pool"], a["ring"], a["ring_base"])
    fold = la.kda_ring_fold if kda else la.gdn_ring_fold
    with pytest.raises(ValueError, match="q"):
        fold(torch.ones(B, dtype=i32), a["slots"], a["ssm_pool"], a["ring"], a["ring_base"],
             q=torch.zeros(B, Hv, D, dtype=f32))                       # ring is bf16
    with pytest.raises(ValueError, match="GPU"):
        fold(torch.ones(B, dtype=i32), a["slots"], a["ssm_pool"], a["ring"], a["ring_base"])


def test_scatter_and_track_copy_reject():
    pool = torch.zeros(P + 1, 3, C, dtype=bf16)
    spool = torch.zeros(P + 1, Hv, D, D, dtype=bf16)
    win = torch.zeros(B, 4, 3, C, dtype=bf16)
    slots = torch.arange(1, B + 1, dtype=i32)
    with pytest.raises(ValueError, match="step"):
        la.conv_window_scatter(win, slots, torch.zeros(B, dtype=torch.int64), pool)
    with pytest.raises(ValueError, match="windows"):
        la.conv_window_scatter(win.float(), slots, torch.zeros(B, dtype=i32), pool)
    with pytest.raises(ValueError, match="GPU"):
        la.conv_window_scatter(win, slots, torch.zeros(B, dtype=i32), pool)
    with pytest.raises(ValueError, match="dst"):
        la.state_track_copy(slots, slots[:2], pool, spool)
    with pytest.raises(ValueError, match="GPU"):
        la.state_track_copy(slots, slots, pool, spool)
