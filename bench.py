"""Benchmark of the recurrent-state hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Headline (`value`): KDA decode tokens/s on the 69-layer stack -- 128
requests, 96 heads, d_k = d_v = 128, bf16 state and conv state in per-layer
pools of 129 rows, per-channel decay.  One step = one fused decode launch
(short conv + SiLU + L2 norm + gated delta rule) per layer, 69 launches,
for the 128-request batch: 128 tokens.  The step is captured once as a HIP
graph; W untimed replays, then exactly K timed replays, each bracketed by
HIP events on the launch stream.  `value` = 128 K / (elapsed over the K
replays); the per-step median is reported beside it.  The layer inputs are
generated once and reused every step while the states evolve; inputs and
pools (31 GB) are resident in HBM before the timed region starts.

`roofline` is the decode kernel's at that shape: algorithmic bytes per
launch (every state row read and written once, the conv history read and
written, x, gates, output and weights moved once) over the average launch
time (step time / 69), against 8 TB/s; `traffic` is the HBM bytes per launch
measured with rocprofv3 counters (FETCH_SIZE and WRITE_SIZE scaled by a
plain copy's readings) when they were taken for the current kernel source.
`cpu_baseline` is the fp64 C oracle on a bounded sample of the same workload
(see cpu_decode_rate), on every host core and single-threaded.

`extra` holds the other workloads, each timed the same way (median of at
least 20 graph replays) with its own roofline and CPU baseline: the
single-layer KDA decode (64 requests x 12 heads, pools rotated over >= 1 GiB
of copies so nothing is served from the on-die cache), the 48-layer GDN fp32
decode (16 q/k heads shared by 32 value heads, 256 requests), the chunked
prefill (one 13,600-token sequence in 6,144 / 6,144 / 1,312-token scheduler
chunks plus eight packed 4,096-token sequences, H = 12; GDN with 16/32
heads) and the speculative-decode calls.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_recurrent_amd import binding as la  # noqa: E402
from linear_attention_recurrent_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFS = 157.3
MFMA_BF16_PEAK_TFS = 2500.0
# algorithmic matrix work of the chunked prefill per token and value head
# (blocks of 64: A, P, T RHS, P D at 64^2 d each, (K Gamma) S^T, (Q Gamma) S^T
# and D^T K at 64 d^2 each; 10.5 MFLOP per 64-token block)
PREFILL_ALG_FLOPS_PER_TOKEN_HEAD = (8 * 64 * 64 * 128 + 6 * 64 * 128 * 128) / 64
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"# bench: {msg}", file=sys.stderr, flush=True)


def esize(dt: str) -> int:
    return 2 if dt == "bf16" else 4


def decode_bytes(sh: synth.DecodeShape) -> int:
    """Algorithmic HBM bytes of one fused decode launch."""
    B, C = sh.B, sh.C
    state = 2 * B * sh.Hv * sh.dv * sh.dk * esize(sh.state)
    conv = 2 * B * 3 * C * esize(sh.conv)
    x = B * C * esize(sh.io)
    g = B * sh.Hv * (sh.dk if sh.kda else 1) * 4
    beta = B * sh.Hv * 4
    out = B * sh.Hv * sh.dv * esize(sh.io)
    w = C * 4 * 4
    return state + conv + x + g + beta + out + w + B * 4


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_recurrent_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ("decode_kernel.h", "la_device.h")
PREFILL_SOURCES = ("prefill.hip", "la_device.h")


def measured_traffic(tag: str, src_hash: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes (per launch, or the `key` given) from profiles/<tag>.traffic.txt,
    or None when that summary is absent or was taken for a different kernel
    source."""
    path = os.path.join(PROFILES, f"{tag}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash or key not in kv:
        return None
    return float(kv[key])


def events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


# ---------------------------------------------------------------- decode ----

def run_decode(sh, inp, out, layer=None):
    fn = la.kda_decode_step if sh.kda else la.gdn_decode_step
    pick = (lambda t: t[layer]) if layer is not None else (lambda t: t)
    fn(pick(inp["x"]), pick(inp["g"]), pick(inp["beta"]), inp["slots"], pick(inp["ssm_pool"]),
       Hqk=sh.Hqk, conv_w=pick(inp["w"]), conv_pool=pick(inp["conv_pool"]), out=out)


def time_replays(launch_all, n_launch, reps, warmup):
    """Captures `launch_all` (n_launch kernel launches) as a HIP graph,
    replays it `warmup` times untimed, then exactly `reps` times, each replay
    between two HIP events on the current stream (the stream the library
    launches on).  Returns per-launch times: the mean over the whole timed
    span (ms_per_launch), the median and extremes over replays."""
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_all()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) / n_launch
    total = ev[0].elapsed_time(ev[reps])
    del graph
    return {"ms_per_launch": total / (reps * n_launch), "median_ms_per_launch": float(np.median(per)),
            "min_ms_per_launch": float(per.min()), "max_ms_per_launch": float(per.max()),
            "replays": reps, "launches_per_replay": n_launch, "elapsed_ms": total}


def decode_stack(sh, layers, steps, warmup, seed, dev):
    """`layers` stacked layers, each with its own pools and inputs; one step =
    one decode launch per layer (one graph replay).  Returns a dict."""
    L, B, C = layers, sh.B, sh.C
    log(f"decode stack: {L} layers, B={B}, H_qk={sh.Hqk}, H_v={sh.Hv}, {sh.state} state")
    n_ssm = (sh.P + 1) * sh.Hv * sh.dv * sh.dk
    n_conv = (sh.P + 1) * 3 * C
    ssm = torch.empty((L, sh.P + 1, sh.Hv, sh.dv, sh.dk), dtype=synth.TORCH_DTYPE[sh.state],
                      device=dev)
    conv = torch.empty((L, sh.P + 1, 3, C), dtype=synth.TORCH_DTYPE[sh.conv], device=dev)
    for l in range(L):
        if l % 8 == 0:
            log(f"decode stack: generating layer {l} of {L}")
        ssm[l].view(-1).copy_(synth.normal_torch(seed + l, synth.S_SSM, n_ssm, dev,
                                                 synth.TORCH_DTYPE[sh.state]))
        conv[l].view(-1).copy_(synth.normal_torch(seed + l, synth.S_CONV, n_conv, dev,
                                                  synth.TORCH_DTYPE[sh.conv]))
    gsz = B * sh.Hv * (sh.dk if sh.kda else 1)
    inp = dict(
        x=synth.normal_torch(seed, synth.S_X, L * B * C, dev, synth.TORCH_DTYPE[sh.io]).view(L, B, C),
        w=(0.5 * synth.normal_torch(seed, synth.S_W, L * C * 4, dev, torch.float64)).to(
            torch.float32).view(L, C, 4),
        g=synth.log_decay_torch(seed, synth.S_G, L * gsz, dev).view(
            (L, B, sh.Hv, sh.dk) if sh.kda else (L, B, sh.Hv)),
        beta=synth.beta_gate_torch(seed, synth.S_BETA, L * B * sh.Hv, dev).view(L, B, sh.Hv),
        slots=torch.from_numpy(synth.slot_permutation(seed, synth.S_SLOTS, sh.P)[:B].copy()).to(dev),
        ssm_pool=ssm, conv_pool=conv)
    outs = [torch.empty((B, sh.Hv, sh.dv), dtype=synth.TORCH_DTYPE[sh.io], device=dev)
            for _ in range(L)]
    for l in range(L):
        run_decode(sh, inp, outs[l], layer=l)
    torch.cuda.synchronize()

    def launch_all():
        for l in range(L):
            run_decode(sh, inp, outs[l], layer=l)

    t = time_replays(launch_all, L, steps, warmup)
    step_ms = t["ms_per_launch"] * L
    nbytes = decode_bytes(sh)
    gbs = nbytes / (t["ms_per_launch"] * 1e-3) / 1e9
    del inp, ssm, conv, outs
    torch.cuda.empty_cache()
    return {"tokens_per_s": B / (step_ms * 1e-3),
            "median_tokens_per_s": B / (t["median_ms_per_launch"] * L * 1e-3),
            "ms_per_step": step_ms, "median_ms_per_step": t["median_ms_per_launch"] * L,
            "steps": t["replays"], "warmup": warmup, "layers": L, "batch": B,
            "timing": t,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes,
                         "launch_us": t["ms_per_launch"] * 1e3}}


def decode_single_layer(sh, reps, dev):
    """One decode launch per step at a single layer's shape; the 34 MB
    working set would sit in the on-die cache, so a replay launches the
    decode once on each of n independent pool + input copies (>= 1 GiB in
    all), as consecutive layers of a model would."""
    per_copy = (sh.P + 1) * (sh.Hv * sh.dv * sh.dk + 3 * sh.C) * esize(sh.state)
    n = max(16, -(-(1 << 30) // per_copy))
    log(f"single-layer decode: B={sh.B}, H={sh.Hv}, {n} rotated copies")
    copies = [synth.decode_inputs(sh, 1001 + 7919 * i, dev) for i in range(n)]
    outs = [torch.empty((sh.B, sh.Hv, sh.dv), dtype=synth.TORCH_DTYPE[sh.io], device=dev)
            for _ in copies]
    for i in range(n):
        run_decode(sh, copies[i], outs[i])
    torch.cuda.synchronize()

    def launch_all():
        for i in range(n):
            run_decode(sh, copies[i], outs[i])

    t = time_replays(launch_all, n, reps, 2)
    nbytes = decode_bytes(sh)
    gbs = nbytes / (t["median_ms_per_launch"] * 1e-3) / 1e9
    traffic = measured_traffic("decode_kda_b64_h12_bf16", source_hash(*DECODE_SOURCES))
    del copies, outs
    torch.cuda.empty_cache()
    return {"tokens_per_s": sh.B / (t["median_ms_per_launch"] * 1e-3),
            "us_per_launch": t["median_ms_per_launch"] * 1e3, "batch": sh.B, "heads": sh.Hv,
            "pool_copies_rotated": n, "timing": t,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                         "algorithmic_bytes_per_launch": nbytes}}


# ----------------------------------------------------- speculative decode ----

def spec_bench(dev, D=8, L=16, reps=20):
    """Speculative verify of D draft tokens and the exact commit at the
    single-layer serving shape (64 requests x 12 heads, d=128, bf16 I/O, state,
    conv and ring), plus the tracking copy and the conv-window scatter of the
    same batch.  Pools, rings and inputs are rotated over copies worth >= 1 GiB
    so every call streams from HBM; each call type is replayed from a captured
    HIP graph."""
    sh = synth.DecodeShape(B=64, Hqk=12, Hv=12, dk=128, dv=128, P=80)
    B, H, d, C, P = sh.B, sh.Hv, sh.dk, sh.C, sh.P
    bf = torch.bfloat16
    per_copy = (P + 1) * (H * d * d * 2 + 3 * C * 2 + H * L * (4 * d * 2 + d * 4 + 4))
    n = max(16, -(-(1 << 30) // per_copy))
    log(f"speculative decode: {n} rotated copies")
    copies = []
    for i in range(n):
        seed = 2001 + 7919 * i
        base = synth.decode_inputs(sh, seed, dev)
        copies.append(dict(
            base,
            x=synth.normal_torch(seed, synth.S_X, B * D * C, dev, bf).view(B, D, C),
            g=synth.log_decay_torch(seed, synth.S_G, B * D * H * d, dev).view(B, D, H, d),
            beta=synth.beta_gate_torch(seed, synth.S_BETA, B * D * H, dev).view(B, D, H),
            ring=la.new_ring(P + 1, H, L, d, d, kda=True, dtype=bf, device=dev),
            n_tok=torch.full((B,), D, dtype=torch.int32, device=dev),
            base=torch.zeros(B, dtype=torch.int32, device=dev),
            acc=torch.full((B,), D, dtype=torch.int32, device=dev),
            step=torch.full((B,), D - 1, dtype=torch.int32, device=dev),
            out=torch.empty((B, D, H, d), dtype=bf, device=dev),
            win=torch.empty((B, D, 3, C), dtype=bf, device=dev),
            dst=(base["slots"] % P) + 1,  # another row of the same pool
            q=synth.normal_torch(seed, synth.S_Q, B * H * d, dev, bf).view(B, H, d),
            o1=torch.empty((B, H, d), dtype=bf, device=dev)))
    def verify(c):
        la.kda_verify(c["x"], c["g"], c["beta"], c["slots"], c["n_tok"], c["ssm_pool"], c["ring"],
                      c["base"], Hqk=H, conv_w=c["w"], conv_pool=c["conv_pool"], out=c["out"],
                      windows=c["win"])
    def commit(c):
        la.kda_commit(c["acc"], c["slots"], c["ssm_pool"], c["ring"], c["base"])
    def scatter(c):
        la.conv_window_scatter(c["win"], c["slots"], c["step"], c["conv_pool"])
    def track(c):
        la.state_track_copy(c["slots"], c["dst"], c["conv_pool"], c["ssm_pool"])
    def fold(c):
        la.kda_ring_fold(c["acc"], c["slots"], c["ssm_pool"], c["ring"], c["base"], q=c["q"],
                         out=c["o1"])
    for c in copies:
        verify(c)
    torch.cuda.synchronize()
    res = {"batch": B, "heads": H, "draft_tokens": D, "ring_depth": L, "dtype": "bf16",
           "pool_copies_rotated": n}
    state = B * H * d * d * 2
    ring_step = H * (4 * d * 2 + d * 4 + 4)            # d, k, rawv, rawk, g, beta per request
    nbytes = {
        # state read; x, g, beta read; conv history read; outputs, windows, ring written
        "verify": state + B * D * (C * 2 + H * d * 4 + H * 4) + B * 3 * C * 2 + C * 16
                  + B * D * (H * d * 2 + 3 * C * 2 + ring_step),
        # state read + written; rawk, rawv, g, beta of D steps read
        "commit": 2 * state + B * D * H * (2 * d * 2 + d * 4 + 4),
        "conv_window_scatter": 2 * B * 3 * C * 2,
        # state read + written; d, k, g of D steps read; q read, out written
        "ring_fold": 2 * state + B * D * H * (2 * d * 2 + d * 4) + 2 * B * H * d * 2,
        "state_track_copy": 2 * B * (H * d * d * 2 + 3 * C * 2),
    }
    for name, fn in (("verify", verify), ("commit", commit), ("ring_fold", fold),
                     ("conv_window_scatter", scatter), ("state_track_copy", track)):
        ms = time_replays(lambda: [fn(c) for c in copies], n, reps, 2)["median_ms_per_launch"]
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        res[name] = {"us": ms * 1e3, "roofline": {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes[name]}}
    res["verify"]["draft_tokens_per_s"] = B * D / (res["verify"]["us"] * 1e-6)
    del copies
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------- prefill ----

def prefill_mfma_flops(seqlens, Hv, mode=0, raw_q=False) -> float:
    """Matrix-core flops the two prefill kernels issue for one packed call,
    following their loop structure.  mode 0 (fp32): v_mfma_f32_16x16x4f32,
    2,048 flops each; mode 1 (bf16x3): three v_mfma_f32_16x16x32_bf16 per
    32-deep step, 16,384 flops each (the T-inverse level products stay fp32
    in both modes).  raw_q (GDN, bf16 inputs, mode 1): the chain forms Q S^T
    from the q rows themselves, two products per step instead of three."""
    T = int(sum(seqlens))
    tiles = -(-T // 64)
    if mode == 0:
        # per (tile, head): A and P 10 jobs x 2 x 32; T levels 64; U, W 8 waves x 2 x 48
        intra = tiles * Hv * (640 + 64 + 768) * 2048.0
        per_chain_tile = (4 * 80 + 4 * 32) * 2048.0       # row waves D + O; column waves
    else:
        intra = tiles * Hv * ((240 + 288) * 16384.0 + 64 * 2048.0)
        per_chain_tile = (4 * (26 if raw_q else 30) + 4 * 12) * 16384.0
    chain_tiles = 0
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    for n in range(len(seqlens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            chain_tiles += (b - 1) // 64 - a // 64 + 1
    return intra + chain_tiles * 8 * Hv * per_chain_tile   # eight 16-row state slices per head


def prefill_bench(dev, reps=20, per_graph=10):
    """Chunked KDA prefill, H=12, d=128, bf16 I/O, fp32 state: W1 = one
    13,600-token sequence in 6,144 / 6,144 / 1,312-token calls chained through
    a pool slot; W2 = eight 4,096-token sequences packed in one call.  Each call
    is the varlen short conv over the projections (C = 12 * 384) followed by
    the chunked prefill on q|k|v views of its output."""
    H, D = 12, 128
    C = 3 * H * D
    seed = 1005
    log("prefill: generating inputs")

    def make(T):
        x = synth.normal_torch(seed + T, synth.S_X, T * C, dev, torch.bfloat16).view(T, C)
        g = synth.log_decay_torch(seed + T, synth.S_G, T * H * D, dev).view(T, H, D)
        beta = synth.beta_gate_torch(seed + T, synth.S_BETA, T * H, dev).view(T, H)
        return x, g, beta

    w = (0.5 * synth.normal_torch(seed, synth.S_W, C * 4, dev, torch.float64)).to(
        torch.float32).view(C, 4)
    conv_pool = torch.zeros((10, 3, C), dtype=torch.bfloat16, device=dev)
    ssm_pool = torch.zeros((10, H, D, D), dtype=torch.float32, device=dev)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    x1, g1, b1 = make(13600)
    x2, g2, b2 = make(8 * 4096)
    cuts = [0, 6144, 12288, 13600]
    calls = []  # (x, g, beta, cu, slot_in, slot_out, seqlens)
    for c in range(3):
        a, b = cuts[c], cuts[c + 1]
        calls.append((x1[a:b], g1[a:b], b1[a:b], i32([0, b - a]), i32([-1 if c == 0 else c]),
                      i32([c + 1]), (b - a,)))
    calls.append((x2, g2, b2, i32(list(range(0, 8 * 4096 + 1, 4096))), i32([-1] * 8),
                  i32(list(range(2, 10))), (4096,) * 8))
    ws = torch.empty(la.kda_prefill_workspace_bytes(8, 8 * 4096, H, H, D, D), dtype=torch.uint8,
                     device=dev)
    ys = [torch.empty((cl[0].shape[0], C), dtype=torch.bfloat16, device=dev) for cl in calls]
    outs = [torch.empty((cl[0].shape[0], H, D), dtype=torch.bfloat16, device=dev) for cl in calls]

    def conv(i):
        x, g, beta, cu, si, so, _ = calls[i]
        la.shortconv_prefill(x, cu, si, so, w, conv_pool, y=ys[i])

    def chunk(i, mode=0):
        x, g, beta, cu, si, so, _ = calls[i]
        y = ys[i]
        q = y[:, :H * D].unflatten(1, (H, D))
        k = y[:, H * D:2 * H * D].unflatten(1, (H, D))
        v = y[:, 2 * H * D:].unflatten(1, (H, D))
        la.kda_prefill_chunked(q, k, v, g, beta, cu, si, so, ssm_pool, out=outs[i], workspace=ws,
                               mode=mode)

    def fused(i, mode=1):
        x, g, beta, cu, si, so, _ = calls[i]
        la.kda_prefill_conv(x, g, beta, cu, si, so, ssm_pool, Hqk=H, conv_w=w,
                            conv_pool=conv_pool, out=outs[i], workspace=ws, mode=mode)

    def run_all(mode):
        for i in range(4):
            conv(i)
            chunk(i, mode)

    res_modes = {}
    for mode in (0, 1):
        log(f"prefill: timing mode {mode}")
        run_all(mode)  # every slot a call reads now holds its predecessor's hand-off
        torch.cuda.synchronize()
        t_conv = [time_replays(lambda i=i: [conv(i) for _ in range(per_graph)], per_graph, reps,
                               2)["median_ms_per_launch"] for i in range(4)]
        t_chunk = [time_replays(lambda i=i: [chunk(i, mode) for _ in range(per_graph)], per_graph,
                                reps, 2)["median_ms_per_launch"] for i in range(4)]
        res_modes[mode] = (t_conv, t_chunk)
    # the conv fused into the prefill's loads (one call per chunk, bf16x3)
    log("prefill: timing the fused conv")
    t_fused = [time_replays(lambda i=i: [fused(i) for _ in range(per_graph)], per_graph, reps,
                            2)["median_ms_per_launch"] for i in range(4)]
    # primary: the bf16x3 mode (pre-split bf16 operands, fp32 accumulation;
    # meets 1e-4 on the fp32 end state like the fp32 mode)
    t_conv, t_chunk = res_modes[1]
    w1_ms = sum(t_conv[:3]) + sum(t_chunk[:3])
    w2_ms = t_conv[3] + t_chunk[3]
    T_all = 13600 + 8 * 4096
    alg = PREFILL_ALG_FLOPS_PER_TOKEN_HEAD * T_all * H
    flops = sum(prefill_mfma_flops(cl[6], H, 1) for cl in calls)
    chunk_ms = sum(t_chunk)
    tf = alg / (chunk_ms * 1e-3) / 1e12
    tf_issued = flops / (chunk_ms * 1e-3) / 1e12
    conv_bytes = sum(2 * cl[0].numel() * 2 for cl in calls)  # x read + y written, bf16
    conv_gbs = conv_bytes / (sum(t_conv) * 1e-3) / 1e9
    # HBM view: the algorithmic bytes (q, k, v, g, beta read and the outputs
    # written once per token-head, each sequence's state read and written
    # once per call) against the kernels' measured traffic
    alg_bytes = T_all * H * (3 * D * 2 + D * 4 + 4 + D * 2) + 11 * H * D * D * 4 * 2
    traffic = measured_traffic("prefill_kda_h12_13600x3chunks_8x4096", source_hash(*PREFILL_SOURCES),
                               "hbm_bytes_per_call_set")
    hbm_gbs = traffic / (chunk_ms * 1e-3) / 1e9 if traffic else None
    f_conv, f_chunk = res_modes[0]
    f_w1 = sum(f_conv[:3]) + sum(f_chunk[:3])
    f_w2 = f_conv[3] + f_chunk[3]
    f_flops = sum(prefill_mfma_flops(cl[6], H, 0) for cl in calls)
    f_tf = alg / (sum(f_chunk) * 1e-3) / 1e12
    res = {
        "tokens_per_s": T_all / ((w1_ms + w2_ms) * 1e-3),
        "w1_13600_tokens_per_s": 13600 / (w1_ms * 1e-3),
        "w2_8x4096_tokens_per_s": 8 * 4096 / (w2_ms * 1e-3),
        "ms": {"w1_total": w1_ms, "w2_total": w2_ms, "conv_calls": t_conv,
               "chunked_calls": t_chunk},
        "mode": "bf16x3 (operands split into bf16 hi + lo, three v_mfma_f32_16x16x32_bf16 "
                "per 32-deep step, fp32 accumulation)",
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFS,
                     "algorithmic_flops": alg,
                     "issued_mfma_flops": flops, "issued_tflops": tf_issued,
                     "issued_frac": tf_issued / MFMA_BF16_PEAK_TFS,
                     "note": "chunked-prefill kernels only (conv separate); achieved = "
                             "algorithmic flops (164 kFLOP per token-head) / time; issued "
                             "flops count the three bf16 products of every split step; the "
                             "chain over 213 dependent blocks of the 13,600-token sequence "
                             "bounds W1",
                     "hbm_view": {"bound": "hbm", "algorithmic_bytes": alg_bytes, "traffic": traffic,
                                  "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": hbm_gbs / HBM_PEAK_GBS if hbm_gbs else None,
                                  "traffic_over_algorithmic": traffic / alg_bytes if traffic else None,
                                  "note": "measured HBM bytes of kernel 1 and the chain over the four "
                                          "calls (rocprofv3 FETCH_SIZE / WRITE_SIZE) per chunked time; "
                                          "the excess over the algorithmic bytes is the workspace "
                                          "kernel 1 writes and the chain reads back"}},
        "conv_roofline": {"bound": "hbm", "achieved": conv_gbs, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": conv_gbs / HBM_PEAK_GBS},
        "fp32_mode": {
            "tokens_per_s": T_all / ((f_w1 + f_w2) * 1e-3),
            "w1_13600_tokens_per_s": 13600 / (f_w1 * 1e-3),
            "w2_8x4096_tokens_per_s": 8 * 4096 / (f_w2 * 1e-3),
            "chunked_calls_ms": f_chunk,
            "roofline": {"bound": "mfma", "achieved": f_tf, "peak": MFMA_FP32_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": f_tf / MFMA_FP32_PEAK_TFS,
                         "algorithmic_flops": alg, "issued_mfma_flops": f_flops,
                         "issued_frac": f_flops / (sum(f_chunk) * 1e-3) / 1e12 / MFMA_FP32_PEAK_TFS},
        },
        "fused_conv": {
            "tokens_per_s": T_all / (sum(t_fused) * 1e-3),
            "w1_13600_tokens_per_s": 13600 / (sum(t_fused[:3]) * 1e-3),
            "w2_8x4096_tokens_per_s": 8 * 4096 / (t_fused[3] * 1e-3),
            "calls_ms": t_fused,
            "speedup_vs_separate_conv": (w1_ms + w2_ms) / sum(t_fused),
            "note": "kda_prefill_conv: the short conv inside the prefill's loads, bf16x3 mode",
        },
        "timing": f"median over {reps} replays of a captured HIP graph of {per_graph} copies "
                  "of each call; W1 = its three conv and three chunked calls",
    }
    del x1, x2, g1, g2, b1, b2, ws, ys, outs, calls
    torch.cuda.empty_cache()
    return res


def gdn_prefill_bench(dev, reps=20, per_graph=10):
    """Chunked GDN prefill with the GDN decode configuration's heads (16 q/k
    heads shared by 32 value heads, d=128), bf16 I/O, fp32 state, scalar
    gate: eight 4,096-token sequences packed in one call, fresh states to
    eight slots.  q, k, v are post-conv inputs (the chunked call alone), both
    precision modes, each call replayed from a captured HIP graph."""
    Hqk, Hv, D = 16, 32, 128
    sh = synth.PrefillShape(seqlens=(4096,) * 8, Hqk=Hqk, Hv=Hv, dk=D, dv=D, kda=False)
    log("GDN prefill: generating inputs")
    inp = synth.prefill_inputs(sh, 1007, dev)
    pool = torch.zeros((9, Hv, D, D), dtype=torch.float32, device=dev)
    si = torch.full((8,), -1, dtype=torch.int32, device=dev)
    so = torch.arange(1, 9, dtype=torch.int32, device=dev)
    out = torch.empty((sh.T, Hv, D), dtype=torch.bfloat16, device=dev)
    res = {}
    for mode, name in ((1, "bf16x3"), (0, "fp32")):
        log(f"GDN prefill: timing {name} mode")
        ws = torch.empty(la.gdn_prefill_workspace_bytes(8, sh.T, Hqk, Hv, D, D, mode),
                         dtype=torch.uint8, device=dev)

        def call():
            la.gdn_prefill_chunked(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["cu_seqlens"], si, so, pool, out=out, workspace=ws,
                                   mode=mode)

        call()
        torch.cuda.synchronize()
        ms = time_replays(lambda: [call() for _ in range(per_graph)], per_graph, reps,
                          2)["median_ms_per_launch"]
        flops = prefill_mfma_flops(sh.seqlens, Hv, mode, raw_q=mode == 1 and sh.io == "bf16")
        alg = PREFILL_ALG_FLOPS_PER_TOKEN_HEAD * sh.T * Hv
        peak = MFMA_BF16_PEAK_TFS if mode else MFMA_FP32_PEAK_TFS
        tf = alg / (ms * 1e-3) / 1e12
        res[name] = {"tokens_per_s": sh.T / (ms * 1e-3), "ms": ms,
                     "roofline": {"bound": "mfma", "achieved": tf, "peak": peak,
                                  "unit": "TFLOP/s", "frac": tf / peak, "algorithmic_flops": alg,
                                  "issued_mfma_flops": flops,
                                  "issued_frac": flops / (ms * 1e-3) / 1e12 / peak}}
        del ws
    res["workload"] = "gdn_prefill_8x4096_hqk16_hv32"
    del inp, pool, out
    torch.cuda.empty_cache()
    return res


def host_threads() -> int:
    """Worker threads for the all-core CPU baselines: every logical CPU the
    process may use, capped at 16 (a GPU machine's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _repeat(fn, budget_s):
    """Runs fn() until budget_s seconds have passed; returns (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def _threaded(fn, threads, budget_s):
    """fn() repeated for budget_s seconds on each of `threads` threads at once
    (the oracle's C calls release the interpreter lock); returns (calls,
    seconds of the slowest thread)."""
    import threading
    res = [None] * threads

    def work(i):
        res[i] = _repeat(fn, budget_s)

    ts = [threading.Thread(target=work, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(r[0] for r in res), max(r[1] for r in res)


def cpu_decode_rate(sh, layers, seed, b_sample, budget_s=8.0):
    """The fp64 C oracle (token by token, as it stands) on a bounded sample of
    a decode workload: one layer's decode step for b_sample requests x all
    value heads, with the workload's shapes, dtypes and value distributions,
    repeated for budget_s seconds single-threaded and then on every host
    core.  A token of the workload needs that update for all `layers`
    layers, so tokens/s = requests updated per second / layers (an
    extrapolation from the sample, labelled as such)."""
    import oracle
    sub = synth.DecodeShape(B=b_sample, Hqk=sh.Hqk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, P=b_sample,
                            kda=sh.kda, io=sh.io, state=sh.state, conv=sh.conv)
    inp = synth.decode_inputs(sub, seed, "cpu")
    f = {k: v.to(torch.float64).numpy() if v.is_floating_point() else v.numpy()
         for k, v in inp.items()}

    def step():
        oracle.decode(f["x"], f["w"], None, f["conv_pool"], f["g"], f["beta"], f["slots"],
                      f["ssm_pool"], Hqk=sub.Hqk, Hv=sub.Hv, dk=sub.dk, dv=sub.dv, kda=sub.kda,
                      conv_dtype=sub.conv, state_dtype=sub.state, io_dtype=sub.io)

    step()  # builds / loads the oracle before any thread starts
    reps1, el1 = _repeat(step, budget_s)
    nt = host_threads()
    repsn, eln = _threaded(step, nt, budget_s)
    one = b_sample * reps1 / el1 / layers
    alln = b_sample * repsn / eln / layers
    what = (f"fp64 C oracle, token by token: one layer's decode step for {b_sample} requests x "
            f"{sh.Hv} value heads (d={sh.dk}, {sh.state} state), repeated for {budget_s:.0f} s; "
            f"tokens/s = requests updated per s / {layers} layers (extrapolated from the sample)")
    return {"value": alln, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"{what}; {repsn} steps on {nt} threads in {eln:.1f} s",
            "extrapolated": True,
            "single_thread": {"value": one, "cores": 1, "steps": reps1, "seconds": el1},
            "host": {"logical_cpus": os.cpu_count(), "machine": platform.machine(),
                     "processor": platform.processor()}}


def cpu_prefill_rate(tokens=6144, budget_s=8.0):
    """The fp64 C oracle's prefill of the first `tokens`-token scheduler chunk
    of the long-sequence workload (H=12, d=128), repeated for budget_s
    seconds: single-threaded over all 12 heads, and on every host core with
    each thread running one head (tokens/s of the 12-head workload =
    head-tokens per s / 12)."""
    import oracle
    H, D = 12, 128
    sh = synth.PrefillShape(seqlens=(tokens,), Hqk=H, Hv=H, dk=D, dv=D)
    inp = synth.prefill_inputs(sh, 77, "cpu")
    f = {k: v.to(torch.float64).numpy() for k, v in inp.items() if k != "cu_seqlens"}
    pool = np.zeros((2, H, D, D))

    def all_heads():
        oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], [0, tokens], [-1], [1], pool)

    one_head = {k: np.ascontiguousarray(v[:, :1]) for k, v in f.items()}
    pool1 = np.zeros((2, 1, D, D))

    def head():
        oracle.prefill(one_head["q"], one_head["k"], one_head["v"], one_head["g"],
                       one_head["beta"], [0, tokens], [-1], [1], pool1)

    head()
    reps1, el1 = _repeat(all_heads, budget_s)
    nt = host_threads()
    repsn, eln = _threaded(head, nt, budget_s)
    return {"value": tokens * repsn / eln / H, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"fp64 C oracle, token by token: the first {tokens}-token scheduler chunk "
                      f"of the 13,600-token sequence; {nt} threads each running one head "
                      f"({repsn} head-calls in {eln:.1f} s; tokens/s = head-tokens per s / {H})",
            "single_thread": {"value": tokens * reps1 / el1, "cores": 1, "calls": reps1,
                              "seconds": el1, "sample": "all 12 heads per call"}}


def copy_calibration(dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, run under rocprofv3 --pmc to scale
    the FETCH_SIZE / WRITE_SIZE counters (each launch reads and writes
    `nbytes`)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_calibration_bytes": nbytes, "ms": ms,
                      "gbs_rw": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def copy_reference(dev, same_size_bytes, big_bytes=2 << 30):
    """Plain device copies as the practical HBM ceiling: one of big_bytes each
    way (4 GiB moved), and one the size of a decode launch (half its bytes
    each way) replayed over 16 rotated buffer pairs from a HIP graph, as the
    decode is timed."""
    src = torch.empty(big_bytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    big_gbs = 2 * big_bytes / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9
    del src, dst
    half = (same_size_bytes // 2 + 15) // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device=dev).fill_(1),
              torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(16)]

    def launch_all():
        for a, b in pairs:
            b.copy_(a)

    ms = time_replays(launch_all, len(pairs), 20, 2)["median_ms_per_launch"]
    small_gbs = 2 * half / (ms * 1e-3) / 1e9
    del pairs
    torch.cuda.empty_cache()
    return big_gbs, small_gbs, ms


BASELINE_METRIC = "KDA decode tokens/s + achieved HBM GB/s (% peak); chunked-prefill tokens/s"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed decode steps (one step = 69 layer launches, 128 tokens)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (PMC counter scaling)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the chunked-prefill workloads (for counter profiles)")
    ap.add_argument("--single-layer-only", action="store_true",
                    help="only the single-layer KDA decode, 64 requests x 12 heads (for counter "
                         "profiles)")
    ap.add_argument("--layers", type=int, default=69,
                    help="layers of the headline stack (69; fewer only for counter passes, "
                         "whose per-launch figures do not depend on it)")
    ap.add_argument("--reps", type=int, default=20,
                    help="graph replays timed per extra workload (median reported)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    la.load_library()
    if args.single_layer_only:
        s2 = synth.DecodeShape(B=64, Hqk=12, Hv=12, dk=128, dv=128, P=80)
        print(json.dumps({"kda_decode_single_layer_b64_h12": decode_single_layer(s2, args.reps, dev)}),
              flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"kda_prefill_chunked_h12": prefill_bench(dev, args.reps),
                          "gdn_prefill_chunked_hqk16_hv32": gdn_prefill_bench(dev, args.reps)}),
              flush=True)
        return
    sh = synth.DecodeShape(B=128, Hqk=96, Hv=96, dk=128, dv=128, P=128)
    layers = args.layers
    log(f"headline: KDA decode, {layers} layers, {args.steps} timed steps after {args.warmup}")
    st = decode_stack(sh, layers, args.steps, args.warmup, 1002, dev)
    nbytes = decode_bytes(sh)
    traffic = measured_traffic("decode_kda_69layers_h96_b128_bf16", source_hash(*DECODE_SOURCES))
    res = {
        "metric": BASELINE_METRIC,
        "value": st["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": st["steps"],
        "warmup": args.warmup,
        "ms_per_step": st["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 / Box-Muller draws; random bf16 pools, "
                "g = -softplus(randn), beta = sigmoid(randn))",
        "config": {"workload": "kda_decode_69_layers_h96_b128", "layers": layers,
                   "batch": sh.B, "H": sh.Hv, "d_k": sh.dk, "d_v": sh.dv,
                   "state_dtype": sh.state, "conv_dtype": sh.conv, "io_dtype": sh.io,
                   "pool_rows_per_layer": sh.P + 1, "conv_kernel": 4,
                   "tokens_per_step": sh.B},
        "median_tokens_per_s": st["median_tokens_per_s"],
        "median_ms_per_step": st["median_ms_per_step"],
        "roofline": dict(st["roofline"], traffic=traffic,
                         kernel="decode_kernel<128, bf16 state, bf16 io, bf16 conv, KDA, G=1>"),
        "timing": dict(st["timing"], method="one HIP graph of the 69 layer launches; W untimed "
                       "replays, then K replays each between HIP events on the launch stream"),
    }
    big_gbs, small_gbs, small_ms = copy_reference(dev, nbytes)
    res["roofline"]["copy_reference"] = {
        "copy_4gib_gbs": big_gbs, "frac_of_copy_4gib": res["roofline"]["achieved"] / big_gbs,
        "copy_same_size_gbs": small_gbs, "copy_same_size_ms": small_ms,
        "frac_of_copy_same_size": res["roofline"]["achieved"] / small_gbs,
        "note": "plain torch device copies on the same box: 2 GiB each way, and one decode "
                "launch's bytes (half each way) rotated over 16 buffer pairs under graph replay"}
    extra = {}
    if not args.no_extra:
        s2 = synth.DecodeShape(B=64, Hqk=12, Hv=12, dk=128, dv=128, P=80)
        extra["kda_decode_single_layer_b64_h12"] = decode_single_layer(s2, args.reps, dev)
        s4 = synth.DecodeShape(B=256, Hqk=16, Hv=32, dk=128, dv=128, P=256, kda=False, io="fp32",
                               state="fp32", conv="fp32")
        extra["gdn_decode_48_layers_fp32_b256"] = decode_stack(s4, 48, args.reps, 2, 1003, dev)
        log("prefill")
        extra["kda_prefill_chunked_h12"] = prefill_bench(dev, args.reps)
        extra["gdn_prefill_chunked_hqk16_hv32"] = gdn_prefill_bench(dev, args.reps)
        extra["kda_speculative_b64_h12_d8"] = spec_bench(dev, reps=args.reps)
    if not args.no_cpu:
        log("CPU oracle baselines")
        res["cpu_baseline"] = cpu_decode_rate(sh, layers, 1002, b_sample=8)
        if extra:
            extra["kda_decode_single_layer_b64_h12"]["cpu_baseline"] = cpu_decode_rate(
                s2, 1, 1001, b_sample=16)
            extra["gdn_decode_48_layers_fp32_b256"]["cpu_baseline"] = cpu_decode_rate(
                s4, 48, 1003, b_sample=8)
            extra["kda_prefill_chunked_h12"]["cpu_baseline"] = cpu_prefill_rate()
    res["extra"] = extra
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
