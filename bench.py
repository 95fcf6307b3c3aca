"""Benchmark of the recurrent-state hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Headline: KDA decode at the single-layer serving shape (64 requests, 12 heads,
d_k = d_v = 128, bf16 state in an 80-slot pool, bf16 conv state, per-channel
decay): one step = one fused decode launch (conv + SiLU + L2 norm + gated
delta rule) for the 64-request batch.  To keep the 34 MB working set out of
the 256 MB on-die cache, the K timed steps rotate over R independent copies of
the pools and inputs (R * 34 MB >= 1 GB), as consecutive layers of a model do.
`value` is tokens/s = 64 * K / elapsed.  Inputs are resident in HBM before the
timed region starts.

The JSON line also carries the decode kernel's roofline (algorithmic bytes per
launch / average launch time, against 8 TB/s), the HBM traffic measured with
rocprofv3 counters when it was taken for the current kernel source, and the
fp64 CPU oracle's rate on a bounded sample of the same workload.  `extra`
holds the other configurations (69-layer KDA decode, 48-layer GDN fp32 decode,
chunked prefill).
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
PROFILES = os.path.join(ROOT, "profiles")


def esize(dt: str) -> int:
    return 2 if dt == "bf16" else 4


def decode_bytes(sh: synth.DecodeShape) -> int:
    """Algorithmic HBM bytes of one fused decode launch: every state row read
    and written once, the 3-row conv history read and written, and x, g, beta,
    the output, the conv weights and the slots moved once."""
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


def measured_traffic(tag: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<tag>.traffic.txt), or None when it is absent or was taken for
    a different kernel source."""
    path = os.path.join(PROFILES, f"{tag}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != src_hash or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def make_copies(sh, seed, dev, n):
    return [synth.decode_inputs(sh, seed + 7919 * i, dev) for i in range(n)]


def run_decode(sh, inp, out):
    fn = la.kda_decode_step if sh.kda else la.gdn_decode_step
    fn(inp["x"], inp["g"], inp["beta"], inp["slots"], inp["ssm_pool"], Hqk=sh.Hqk,
       conv_w=inp["w"], conv_pool=inp["conv_pool"], out=out)


def time_decode(sh, copies, steps, warmup):
    """Times `steps` decode launches rotating over the copies.  The rotation
    (one launch per copy) is captured once as a HIP graph and replayed, as a
    serving loop replays its decode graph; `steps` is rounded up to a whole
    number of rotations.  Returns (ms per launch from hipEvents on the replay
    stream, steps timed, eager ms per launch from direct calls)."""
    dev = copies[0]["x"].device
    outs = [torch.empty((sh.B, sh.Hv, sh.dv), dtype=synth.TORCH_DTYPE[sh.io], device=dev)
            for _ in copies]
    n = len(copies)
    for i in range(max(warmup, n)):
        run_decode(sh, copies[i % n], outs[i % n])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager (one ctypes call per launch; includes host launch overhead)
    e0.record(stream)
    for i in range(4 * n):
        run_decode(sh, copies[i % n], outs[i % n])
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / (4 * n)
    # graph replay
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            run_decode(sh, copies[i], outs[i])
    torch.cuda.synchronize()
    reps = -(-steps // n)
    for _ in range(max(1, warmup // n)):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n), reps * n, eager_ms


def copy_calibration(dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, run under rocprofv3 --pmc to scale
    the FETCH_SIZE / WRITE_SIZE counters (each launch reads and writes
    `nbytes`)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_calibration_bytes": nbytes, "ms": ms,
                      "gbs_rw": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def cpu_oracle_decode_rate(sh, seed, budget_s=12.0):
    """The fp64 oracle on the same workload's first-layer inputs, repeated
    until `budget_s` seconds; single-threaded."""
    import oracle
    inp = synth.decode_inputs(sh, seed, "cpu")
    f = {k: v.to(torch.float64).numpy() if v.is_floating_point() else v.numpy()
         for k, v in inp.items()}
    # compact pools holding only the batch's rows (row 0 = padding)
    rows = np.concatenate([[0], f["slots"]])
    f["conv_pool"], f["ssm_pool"] = f["conv_pool"][rows], f["ssm_pool"][rows]
    f["slots"] = np.arange(1, sh.B + 1, dtype=np.int32)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(f["x"], f["w"], None, f["conv_pool"], f["g"], f["beta"], f["slots"],
                      f["ssm_pool"], Hqk=sh.Hqk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, kda=sh.kda,
                      conv_dtype=sh.conv, state_dtype=sh.state, io_dtype=sh.io)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return sh.B * reps / el, reps, el


def headline(args, dev):
    sh = synth.DecodeShape(B=64, Hqk=12, Hv=12, dk=128, dv=128, P=80)
    per_copy = ((sh.P + 1) * (sh.Hv * sh.dv * sh.dk + 3 * sh.C) * 2)
    n_copies = max(16, -(-(1 << 30) // per_copy))
    copies = make_copies(sh, 1001, dev, n_copies)
    ms, steps, eager_ms = time_decode(sh, copies, args.steps, args.warmup)
    nbytes = decode_bytes(sh)
    gbs = nbytes / (ms * 1e-3) / 1e9
    src = source_hash("decode.hip", "la_device.h")
    traffic = measured_traffic("decode_kda_b64_h12_bf16", src)
    res = {
        "metric": "KDA decode tokens/s (single layer, 64 requests, H=12, d=128, bf16 state)",
        "value": sh.B / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller; random state, pools rotated over "
                f"{n_copies} copies)",
        "config": {"workload": "kda_decode_single_layer", "batch": sh.B, "H": sh.Hv,
                   "d_k": sh.dk, "d_v": sh.dv, "state_dtype": sh.state, "pool_slots": sh.P,
                   "conv_kernel": 4, "pool_copies_rotated": n_copies},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "decode_kernel<128, bf16, KDA>",
                     "algorithmic_bytes_per_launch": nbytes},
        "eager_ms_per_step": eager_ms,
        "launch": "HIP graph of one decode launch per pool copy, replayed",
    }
    del copies
    torch.cuda.empty_cache()
    return sh, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (PMC counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    la.load_library()
    print(f"# bench: headline KDA decode, {args.steps} steps after {args.warmup} warmup",
          file=sys.stderr, flush=True)
    sh, res = headline(args, dev)
    extra = {}
    res["extra"] = extra
    if not args.no_cpu:
        print("# bench: CPU oracle baseline", file=sys.stderr, flush=True)
        rate, reps, el = cpu_oracle_decode_rate(sh, 1001)
        res["cpu_baseline"] = {
            "value": rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 C oracle, {reps} full decode steps of the 64-request batch "
                      f"(all 12 heads) in {el:.1f} s, single thread, host "
                      f"{platform.processor() or platform.machine()} x{os.cpu_count()}"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
