"""Python face of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and
its binding) never imports this package, and this package imports nothing from
the product path.

Every function takes numpy arrays holding the exact values of the stored
tensors (any float dtype; they are converted to fp64 without loss), copies the
pools it updates, and returns fresh arrays: calls are pure.  The arithmetic is
in ``oracle.c``; this file marshals arguments, except for ``track_copy`` and
``conv_window_scatter``, which are plain row copies (no arithmetic) written
here with numpy indexing.  Storage dtypes are the strings ``"fp32"``,
``"bf16"`` and ``"fp64"`` (no rounding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DTYPES = {"fp32": 0, "bf16": 1, "fp64": 2}
_lib = None


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (plain -O2, no
    fast-math, no FMA contraction, so every operation rounds as written)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_round.argtypes, lib.orc_round.restype = [D, I], D
    lib.orc_round_array.argtypes, lib.orc_round_array.restype = [P, L, I], None
    lib.orc_shortconv_step.argtypes = [I, I, P, P, P, P, L, I, P, P]
    lib.orc_shortconv_step.restype = None
    lib.orc_recurrent_step.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, L, I, P, I, D, D]
    lib.orc_recurrent_step.restype = I
    lib.orc_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, L, I, P, P, P, P, L, I, P, I, D, D]
    lib.orc_decode.restype = I
    lib.orc_shortconv_prefill.argtypes = [I, I, P, P, P, P, P, P, P, L, I, P, I]
    lib.orc_shortconv_prefill.restype = None
    lib.orc_prefill.argtypes = [I, I, I, I, I, I, P, L, P, L, P, L, P, P, P, P, P, P, L, I, P, I, D, D]
    lib.orc_prefill.restype = I
    lib.orc_verify.argtypes = [I, I, I, P, I, I, I, I, P, P, P, P, L, I, P, P, P, P, L, P, I, P,
                               I, P, P, P, P, P, P, P, D, D]
    lib.orc_verify.restype = I
    lib.orc_commit.argtypes = [I, I, P, I, I, I, P, P, L, I, I, P, P, P, P, P, D]
    lib.orc_commit.restype = I
    lib.orc_ring_fold.argtypes = [I, I, P, I, I, I, P, P, P, L, I, I, P, P, P, P, P, P, I, D, D]
    lib.orc_ring_fold.restype = I
    _lib = lib
    return lib


def _f64(a):
    """Exact fp64 copy of a float array (C-contiguous)."""
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def round_to(x, dtype: str) -> np.ndarray:
    """Round values to a storage dtype (nearest, ties to even)."""
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    _load().orc_round_array(y.ctypes.data, y.size, _DTYPES[dtype])
    return y


def shortconv_step(x, w, bias, conv_pool, slots, conv_dtype="fp32"):
    """One decode token of the short conv + SiLU.

    x [B, C]; w [C, 4]; bias [C] or None; conv_pool [P+1, 3, C]; slots [B].
    Returns (y [B, C] fp64 unrounded, new conv_pool)."""
    x, w, bias, pool, slots = _f64(x), _f64(w), _f64(bias), _f64(conv_pool).copy(), _i32(slots)
    B, C = x.shape
    y = np.empty((B, C))
    _load().orc_shortconv_step(B, C, _ptr(x), _ptr(w), _ptr(bias), _ptr(pool),
                               3 * C, _DTYPES[conv_dtype], _ptr(slots), _ptr(y))
    return y, pool


def recurrent_step(q, k, v, g, beta, slots, ssm_pool, *, kda=True,
                   state_dtype="fp32", io_dtype="fp32", eps=1e-6, scale=1.0):
    """Decode recurrence on already-convolved raw q/k/v.

    q, k [B, Hqk, dk]; v [B, Hv, dv]; g [B, Hv, dk] (KDA) or [B, Hv] (GDN);
    beta [B, Hv]; ssm_pool [P+1, Hv, dv, dk].  Returns (out [B, Hv, dv],
    new ssm_pool)."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    slots, pool = _i32(slots), _f64(ssm_pool).copy()
    B, Hqk, dk = q.shape
    _, Hv, dv = v.shape
    out = np.empty((B, Hv, dv))
    rc = _load().orc_recurrent_step(int(kda), B, Hqk, Hv, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(g), _ptr(beta), _ptr(slots), _ptr(pool),
                                    Hv * dv * dk, _DTYPES[state_dtype], _ptr(out),
                                    _DTYPES[io_dtype], eps, scale)
    if rc != 0:
        raise ValueError("oracle: H_v must be a positive multiple of H_qk")
    return out, pool


def decode(x, w, bias, conv_pool, g, beta, slots, ssm_pool, *, Hqk, Hv, dk, dv,
           kda=True, conv_dtype="fp32", state_dtype="fp32", io_dtype="fp32",
           eps=1e-6, scale=1.0):
    """Full decode step (conv + SiLU + split + L2 norm + recurrence).

    x [B, C] with C = 2*Hqk*dk + Hv*dv ordered [Q | K | V]; w [C, 4] or None
    (then x is already post-conv and conv_pool is left alone).
    Returns (out [B, Hv, dv], new conv_pool, new ssm_pool)."""
    x, w, bias, g, beta = map(_f64, (x, w, bias, g, beta))
    slots = _i32(slots)
    cpool = _f64(conv_pool).copy() if conv_pool is not None else None
    spool = _f64(ssm_pool).copy()
    B, C = x.shape
    assert C == 2 * Hqk * dk + Hv * dv
    out = np.empty((B, Hv, dv))
    rc = _load().orc_decode(int(kda), B, Hqk, Hv, dk, dv, _ptr(x), _ptr(w), _ptr(bias),
                            _ptr(cpool), 3 * C, _DTYPES[conv_dtype], _ptr(g), _ptr(beta),
                            _ptr(slots), _ptr(spool), Hv * dv * dk, _DTYPES[state_dtype],
                            _ptr(out), _DTYPES[io_dtype], eps, scale)
    if rc != 0:
        raise ValueError("oracle: H_v must be a positive multiple of H_qk")
    return out, cpool, spool


def shortconv_prefill(x, cu_seqlens, slot_in, slot_out, w, bias, conv_pool, *,
                      conv_dtype="fp32", io_dtype="fp32"):
    """Short conv + SiLU over packed sequences.  x [T, C]; cu_seqlens [N+1];
    slot_in/slot_out [N] (slot_in < 0: zero history); conv_pool [P+1, 3, C].
    Returns (y [T, C] rounded to io_dtype, new conv_pool)."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    cu, si, so = _i32(cu_seqlens), _i32(slot_in), _i32(slot_out)
    pool = _f64(conv_pool).copy()
    T, C = x.shape
    y = np.empty((T, C))
    _load().orc_shortconv_prefill(len(si), C, _ptr(x), _ptr(cu), _ptr(si), _ptr(so), _ptr(w),
                                  _ptr(bias), _ptr(pool), 3 * C, _DTYPES[conv_dtype], _ptr(y),
                                  _DTYPES[io_dtype])
    return y, pool


def prefill(q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, *, kda=True,
            state_dtype="fp32", io_dtype="fp32", eps=1e-6, scale=1.0):
    """Recurrent-state prefill over packed sequences, token by token.

    q, k [T, Hqk, dk]; v [T, Hv, dv]; g [T, Hv, dk] (KDA) or [T, Hv] (GDN);
    beta [T, Hv]; ssm_pool [P+1, Hv, dv, dk].  Returns (out [T, Hv, dv] rounded
    to io_dtype, new ssm_pool)."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu, si, so = _i32(cu_seqlens), _i32(slot_in), _i32(slot_out)
    pool = _f64(ssm_pool).copy()
    T, Hqk, dk = q.shape
    _, Hv, dv = v.shape
    out = np.empty((T, Hv, dv))
    rc = _load().orc_prefill(int(kda), len(si), Hqk, Hv, dk, dv, _ptr(q), Hqk * dk, _ptr(k),
                             Hqk * dk, _ptr(v), Hv * dv, _ptr(g), _ptr(beta), _ptr(cu),
                             _ptr(si), _ptr(so), _ptr(pool), Hv * dv * dk,
                             _DTYPES[state_dtype], _ptr(out), _DTYPES[io_dtype], eps, scale)
    if rc != 0:
        raise ValueError("oracle: H_v must be a positive multiple of H_qk")
    return out, pool


# ------------------------------------------------------ speculative decode --

def new_ring(num_rows, Hv, L, dk, dv, kda=True):
    """An empty ReplaySSM ring (zeros): per pool row, per value head, L steps
    of d [dv], k [dk], g [dk] (KDA) or [1] (GDN), rawv [dv], rawk [dk], and
    beta [] (scalar)."""
    return {"d": np.zeros((num_rows, Hv, L, dv)), "k": np.zeros((num_rows, Hv, L, dk)),
            "g": np.zeros((num_rows, Hv, L, dk if kda else 1)),
            "rawv": np.zeros((num_rows, Hv, L, dv)), "rawk": np.zeros((num_rows, Hv, L, dk)),
            "beta": np.zeros((num_rows, Hv, L))}


def verify(x, w, bias, conv_pool, g, beta, slots, n_tok, ssm_pool, ring, ring_base, *, Hqk,
           Hv, dk, dv, kda=True, conv_dtype="fp32", io_dtype="fp32", eps=1e-6, scale=1.0):
    """Speculative verify of up to D draft tokens per request (x [B, D, C];
    n_tok[b] of them used) from the pool checkpoint; the pools are not
    modified.  Returns (out [B, D, Hv, dv], windows [B, D, 3, C], new ring):
    each step's output, the conv history after each step, and the ring with
    every step's record written at (ring_base[b] + t) mod L."""
    x, w, bias, g, beta = _f64(x), _f64(w), _f64(bias), _f64(g), _f64(beta)
    conv = _f64(conv_pool) if conv_pool is not None else np.zeros((1, 3, 1))
    pool = _f64(ssm_pool)
    slots, n_tok, ring_base = _i32(slots), _i32(n_tok), _i32(ring_base)
    B, D, C = x.shape
    L = ring["d"].shape[2]
    r = {k: _f64(v).copy() for k, v in ring.items()}
    out = np.empty((B, D, Hv, dv))
    windows = np.zeros((B, D, 3, C))
    rc = _load().orc_verify(int(kda), B, D, _ptr(n_tok), Hqk, Hv, dk, dv, _ptr(x), _ptr(w),
                            _ptr(bias), _ptr(conv), conv.shape[1] * conv.shape[2],
                            _DTYPES[conv_dtype], _ptr(g), _ptr(beta), _ptr(slots), _ptr(pool),
                            Hv * dv * dk, _ptr(out), _DTYPES[io_dtype], _ptr(windows), L,
                            _ptr(ring_base), _ptr(r["d"]), _ptr(r["k"]), _ptr(r["g"]),
                            _ptr(r["rawv"]), _ptr(r["rawk"]), _ptr(r["beta"]), eps, scale)
    if rc != 0:
        raise ValueError("oracle: H_v must be a positive multiple of H_qk")
    return out, windows, r


def commit(accepted, slots, ssm_pool, ring, ring_base, *, kda=True, state_dtype="fp32",
           eps=1e-6):
    """Exact commit: replay the first accepted[b] ring steps of each request
    from its pool row and store the result back.  Returns the new pool."""
    pool = _f64(ssm_pool).copy()
    _, Hv, dv, dk = pool.shape
    L = ring["rawv"].shape[2]
    r = {k: _f64(v) for k, v in ring.items()}
    accepted, slots, ring_base = _i32(accepted), _i32(slots), _i32(ring_base)
    _load().orc_commit(int(kda), len(slots), _ptr(accepted), Hv, dk, dv, _ptr(slots), _ptr(pool),
                       Hv * dv * dk, _DTYPES[state_dtype], L, _ptr(ring_base), _ptr(r["g"]),
                       _ptr(r["rawv"]), _ptr(r["rawk"]), _ptr(r["beta"]), eps)
    return pool


def track_copy(conv_pool, ssm_pool, mask, src, dst):
    """State tracking (the state-tracking passage of xxmr.cn/news/181459): for every
    entry i with mask[i] (all when mask is None), pool rows dst[i] of both
    pools become copies of rows src[i].  Returns the new (conv, ssm) pools."""
    conv, ssm = np.array(conv_pool, copy=True), np.array(ssm_pool, copy=True)
    for i in range(len(src)):
        if mask is None or mask[i]:
            conv[dst[i]] = conv_pool[src[i]]
            ssm[dst[i]] = ssm_pool[src[i]]
    return conv, ssm


def conv_window_scatter(conv_pool, windows, mask, slots, step):
    """Commit of the conv history after speculative verify (the
    "intermediate_conv_window" passage of xxmr.cn/news/181459): for every entry b with mask[b] (all
    when mask is None) and 0 <= step[b] < D, pool row slots[b] becomes
    windows[b, step[b]].  Returns the new conv pool."""
    conv = np.array(conv_pool, copy=True)
    D = windows.shape[1]
    for b in range(len(slots)):
        if (mask is None or mask[b]) and 0 <= step[b] < D:
            conv[slots[b]] = windows[b, step[b]]
    return conv


def ring_fold(m, slots, dst, ssm_pool, ring, ring_base, q=None, *, kda=True,
              state_dtype="fp32", io_dtype="fp32", eps=1e-6, scale=1.0):
    """ReplaySSM fast rebuild: S_m from the checkpoint rows slots[b] and the
    ring's (d, k, g) of m[b] steps by the unrolled sum, stored to rows dst[b].
    Returns (new pool, out [B, Hv, dv] = scale S_m q_hat or None)."""
    pool = _f64(ssm_pool).copy()
    _, Hv, dv, dk = pool.shape
    L = ring["d"].shape[2]
    r = {k: _f64(v) for k, v in ring.items()}
    m, slots, dst, ring_base = _i32(m), _i32(slots), _i32(dst), _i32(ring_base)
    q = _f64(q)
    out = np.empty((len(slots), Hv, dv)) if q is not None else None
    _load().orc_ring_fold(int(kda), len(slots), _ptr(m), Hv, dk, dv, _ptr(slots), _ptr(dst),
                          _ptr(pool), Hv * dv * dk, _DTYPES[state_dtype], L, _ptr(ring_base),
                          _ptr(r["d"]), _ptr(r["k"]), _ptr(r["g"]), _ptr(q), _ptr(out),
                          _DTYPES[io_dtype], eps, scale)
    return pool, out
