"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point the header declares, computes pool sizes that reproduce
the pages' printed figures, and rejects bad arguments before any launch."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from linear_attention_recurrent_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "pool_bytes.json")
RING_GOLDEN = os.path.join(ROOT, "tests", "golden", "ring_bytes.json")
HEADER = os.path.join(ROOT, "include", "la.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"kda_decode_step", "gdn_decode_step", "shortconv_update", "shortconv_prefill",
            "kda_prefill_chunked", "la_pool_bytes", "la_last_error", "la_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    hdr = open(HEADER).read()
    assert lib.la_version() == int(re.search(r"#define LA_VERSION (\d+)", hdr).group(1))


def test_pool_bytes_reproduce_printed_figures(lib):
    gold = json.load(open(GOLDEN))
    L, H, d, C = gold["layers"], gold["H_v"], gold["d"], gold["conv_channels"]
    # one row = one request's state across all layers
    ssm, conv = binding.pool_bytes(L, 0, H, d, d, C, "bf16", "bf16")
    pr = gold["per_request"]
    assert ssm == eval(pr["ssm_bytes_product"]) == 27131904
    assert conv == eval(pr["conv_bytes_product"]) == 1907712
    assert round(ssm / 2**20, 1) == pr["ssm_mib"]
    assert round(conv / 2**20, 2) == pr["conv_mib"]
    # the page sums its rounded per-GPU figures over 8 GPUs
    assert round((round(ssm / 2**20, 1) + round(conv / 2**20, 2)) * 8, 1) == pr["tp8_total_mb"]
    for case in gold["allocation_logs"]:
        ssm, conv = binding.pool_bytes(L, case["slots"], H, d, d, C, case["state"], case["conv"])
        assert round(ssm / 2**30, 2) == case["ssm_gib"], case
        assert round(conv / 2**30, 2) == case["conv_gib"], case


def test_ring_bytes_reproduce_printed_figures(lib):
    """The ReplaySSM ring sizes of the pages' allocation log (L = 16, 119
    slots + 1 rows, 69 layers, 12 heads, head dim 128)."""
    gold = json.load(open(RING_GOLDEN))
    got = binding.ring_bytes(gold["layers"], gold["slots"], gold["H_v"], gold["L"], gold["d"],
                             gold["d"], gold["io_dtype"], gold["kda"])
    for name, shape in gold["shapes"].items():
        elem = 2 if name in ("d", "k", "rawv", "rawk") else 4
        assert got[name] == int(np.prod(shape)) * elem, name
        assert round(got[name] / 2**30, 3) == gold["gib"][name], name
    # GDN keeps one gate per head and step
    gdn = binding.ring_bytes(gold["layers"], gold["slots"], gold["H_v"], gold["L"], gold["d"],
                             gold["d"], "bf16", False)
    assert gdn["g"] == got["beta"] and gdn["d"] == got["d"]


def test_ring_bytes_rejects_bad_args(lib):
    out = ctypes.c_int64()
    assert lib.la_ring_bytes(1, -1, 1, 16, 128, 128, 1, 1, ctypes.byref(out), None, None,
                             None) == -1
    assert lib.la_ring_bytes(1, 1, 1, 16, 128, 128, 5, 1, None, None, None, None) == -1


def test_pool_bytes_rejects_bad_args(lib):
    out = ctypes.c_int64()
    assert lib.la_pool_bytes(-1, 1, 1, 1, 1, 1, 0, 0, ctypes.byref(out), None) == -1
    assert b"negative" in lib.la_last_error()
    assert lib.la_pool_bytes(1, 1, 1, 1, 1, 1, 7, 0, ctypes.byref(out), None) == -1


def _decode_args(**over):
    # all-null pointers with B = 4: validation fails before any launch
    a = dict(B=4, Hqk=2, Hv=4, dk=128, dv=128, x=None, io=1, w=None, b=None, cp=None,
             cstride=0, cdt=1, g=None, beta=None, slots=None, rows=9, sp=None,
             sstride=4 * 128 * 128, sdt=1, out=None, eps=1e-6, scale=1.0, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("fn", ["kda_decode_step", "gdn_decode_step"])
def test_decode_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(*_decode_args()) == -1                       # null pointers
    assert b"null pointer" in lib.la_last_error()
    assert f(*_decode_args(Hv=3)) == -1                   # H_v not a multiple of H_qk
    assert f(*_decode_args(dk=96, dv=96)) == -2           # head dim not built
    assert f(*_decode_args(dk=128, dv=64)) == -2
    assert f(*_decode_args(io=5)) == -2                   # unknown dtype
    assert f(*_decode_args(B=-1)) == -1
    assert f(*_decode_args(B=0)) == 0                     # empty batch: no-op
    assert lib.la_last_error() == b""
    fake = ctypes.c_void_p(0x1000)
    mis = ctypes.c_void_p(0x1004)
    good = dict(x=fake, g=fake, beta=fake, slots=fake, sp=fake, out=fake)
    assert f(*_decode_args(**{**good, "x": mis})) == -1   # misaligned
    assert b"aligned" in lib.la_last_error()
    assert f(*_decode_args(**{**good, "sstride": 100})) == -1  # stride too small
    assert f(*_decode_args(**{**good, "w": fake})) == -1  # conv weights without a conv pool


def test_prefill_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    T, H, d = 100, 12, 128
    args = [1, T, H, H, d, d, fake, H * d, fake, H * d, fake, H * d, 1, fake, fake, fake, fake,
            fake, 5, fake, H * d * d, 0, fake, 1e-6, 1.0, 0, None, 0, None]
    need = lib.kda_prefill_workspace_bytes(1, T, H, H, d, d, 0)
    if need:
        assert lib.kda_prefill_chunked(*args) == -3       # workspace missing
        assert b"workspace" in lib.la_last_error()
    bad = list(args)
    bad[4] = bad[5] = 64
    assert lib.kda_prefill_chunked(*bad) == -2            # only d = 128 built
    bad = list(args)
    bad[7] = 10                                           # q stride shorter than a token
    assert lib.kda_prefill_chunked(*bad) == -1
    bad = list(args)
    bad[25] = 2                                           # unknown mode
    assert lib.kda_prefill_chunked(*bad) == -2
    bad = list(args)
    bad[2], bad[3] = 1, 4097                              # H_v beyond the 32-bit output offsets
    bad[11] = 4097 * d
    assert lib.kda_prefill_chunked(*bad) == -2
    assert b"4096" in lib.la_last_error()
    bad = list(args)
    bad[0] = 0                                            # no sequences: no-op
    assert lib.kda_prefill_chunked(*bad) == 0


@pytest.mark.parametrize("fn", ["kda_prefill_conv", "gdn_prefill_conv"])
def test_prefill_conv_validation(lib, fn):
    fake = ctypes.c_void_p(0x1000)
    T, H, d = 100, 12, 128
    C = 3 * H * d
    f = getattr(lib, fn)
    args = [1, T, H, H, d, d, fake, 1, fake, None, fake, 3 * C, 1, fake, fake, fake, fake, fake,
            5, fake, H * d * d, 0, fake, 1e-6, 1.0, 1, None, 0, None]
    if lib.kda_prefill_workspace_bytes(1, T, H, H, d, d, 1):
        assert f(*args) == -3                             # workspace missing
    bad = list(args)
    bad[10] = None                                        # no conv pool
    assert f(*bad) == -1
    bad = list(args)
    bad[11] = 3 * C - 8                                   # conv rows overlap
    assert f(*bad) == -1 and b"conv_slot_stride" in lib.la_last_error()
    bad = list(args)
    bad[12] = 3                                           # unknown conv dtype
    assert f(*bad) == -2
    bad = list(args)
    bad[8] = ctypes.c_void_p(0x1004)                      # misaligned taps
    assert f(*bad) == -1
    bad = list(args)
    bad[0] = 0                                            # no sequences: no-op
    assert f(*bad) == 0


def test_shortconv_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.shortconv_update(4, 64, None, 1, fake, None, fake, 192, 1, 5, fake, fake, None) == -1
    assert lib.shortconv_update(4, 64, fake, 1, fake, None, fake, 100, 1, 5, fake, fake, None) == -1
    assert lib.shortconv_update(0, 64, None, 1, None, None, None, 0, 1, 5, None, None, None) == 0
    assert lib.shortconv_prefill(1, 8, 64, fake, 3, fake, fake, fake, fake, None, fake, 192, 1, 5,
                                 fake, None) == -2


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError, match="no CPU fallback"):
        binding.load_library()


def test_speculative_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    ring = binding.LaRing(16, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    H, d = 2, 128
    C = 3 * H * d

    def verify(**over):
        a = dict(B=4, D=8, n_tok=fake, Hqk=H, Hv=H, dk=d, dv=d, x=fake, io=1, w=None, b=None,
                 cp=None, cstride=0, cdt=1, g=fake, beta=fake, slots=fake, rows=9, sp=fake,
                 sstride=H * d * d, sdt=1, out=fake, win=None, ring=ctypes.byref(ring),
                 base=fake, eps=1e-6, scale=1.0, stream=None)
        a.update(over)
        return lib.kda_verify(*a.values())

    assert verify(x=None) == -1                              # null pointer
    assert verify(dk=64, dv=64) == -2                        # only d = 128 built
    assert verify(D=32) == -1                                # ring shallower than the drafts
    assert b"power of two" in lib.la_last_error()
    bad = binding.LaRing(12, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert verify(ring=ctypes.byref(bad)) == -1              # L not a power of two
    assert verify(ring=None) == -1                           # no ring
    assert verify(w=fake, cp=fake, cstride=3 * C) == -1      # conv without a windows buffer
    assert verify(B=0) == 0
    assert lib.kda_commit(4, fake, H, d, d, fake, 9, fake, H * d * d, 1, 1, None, fake, 1e-6,
                          None) == -1                        # no ring
    assert lib.kda_commit(0, None, H, d, d, None, 9, None, H * d * d, 1, 1, None, None, 1e-6,
                          None) == 0
    assert lib.conv_window_scatter(4, 8, 1, None, fake, fake, fake, fake, 16, 0, 9, None) == -1
    assert b"16 bytes" in lib.la_last_error()                # a 12-byte window
    assert lib.conv_window_scatter(0, 8, C, None, None, None, None, None, 3 * C, 1, 9, None) == 0
    assert lib.state_track_copy(4, None, fake, fake, fake, 40, 36, 1, fake, 64, 64, 0, 9,
                                None) == -1                  # 72-byte conv row
    assert lib.state_track_copy(4, None, fake, None, fake, 48, 48, 1, fake, 64, 64, 0, 9,
                                None) == -1                  # null dst
