"""Seeded synthetic inputs for the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic.  It is a counter-based
random generator plus the value distributions the workloads are defined with:

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state += 0x9E3779B97F4A7C15, then the 64-bit
  finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift 27,
  multiply 0x94D049BB133111EB, xor-shift 31).  Stream ``s`` of seed ``seed``
  starts from state ``mix64((seed << 32) ^ s)``.
* Uniforms in (0, 1]: ``((x >> 11) + 1) * 2**-53``.
* Normals by Box-Muller on consecutive pairs (u1, u2):
  ``r = sqrt(-2 ln u1)``, ``z0 = r cos(2 pi u2)``, ``z1 = r sin(2 pi u2)``.
* Rounding of the fp64 draw: to fp32 (nearest-even), then to bf16 when asked.

The numpy path is the definition.  The torch path computes the same
integers (checked against numpy) and is used to fill multi-GB pools directly
in device memory; its transcendental functions may differ from numpy's in the
last fp64 bit.  Every tensor is drawn from its own stream, so shapes do not
shift one another's values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

# Stream ids: inputs are drawn from these fixed streams.
S_X, S_W, S_G, S_BETA, S_CONV, S_SSM, S_SLOTS, S_Q, S_K, S_V = range(10)


def _mix64_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def _stream_base(seed: int, stream: int) -> int:
    return _mix64_int(((seed & 0xFFFFFFFF) << 32) ^ (stream & 0xFFFFFFFF))


def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


def raw_u64(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """Draws offset .. offset+n-1 of SplitMix64 stream ``stream``."""
    base = np.uint64(_stream_base(seed, stream))
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = base + i * np.uint64(GAMMA)
    return _mix64_np(state)


def uniform(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """Uniform fp64 draws in (0, 1]."""
    x = raw_u64(seed, stream, n, offset)
    return ((x >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53


def normal(seed: int, stream: int, shape) -> np.ndarray:
    """Standard normal fp64 draws of the given shape (Box-Muller pairs)."""
    n = int(np.prod(shape)) if len(shape) else 1
    m = (n + 1) // 2
    u = uniform(seed, stream, 2 * m)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    th = 2.0 * math.pi * u[1::2]
    z = np.empty(2 * m)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    return z[:n].reshape(shape)


# ---------------------------------------------------------------------------
# torch path: same integers, computed with int64 wrap-around arithmetic.
# ---------------------------------------------------------------------------

def _s64(u: int) -> int:
    u &= _MASK
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def raw_u64_torch(seed: int, stream: int, n: int, offset: int = 0, device="cpu") -> torch.Tensor:
    """Same draws as :func:`raw_u64`, as int64 bit patterns."""
    base = _s64(_stream_base(seed, stream))
    i = torch.arange(offset + 1, offset + n + 1, dtype=torch.int64, device=device)
    return _mix64_t(i * _s64(GAMMA) + base)


def normal_torch(seed: int, stream: int, numel: int, device="cpu", dtype=torch.float32,
                 chunk: int = 1 << 26) -> torch.Tensor:
    """Flat tensor of ``numel`` normal draws (same definition as :func:`normal`),
    rounded to ``dtype`` (fp64 kept; else fp64 -> fp32 -> bf16), generated
    chunk by chunk."""
    out = torch.empty(numel, dtype=dtype, device=device)
    m_total = (numel + 1) // 2
    for p0 in range(0, m_total, chunk):
        m = min(chunk, m_total - p0)
        x = raw_u64_torch(seed, stream, 2 * m, 2 * p0, device)
        u = (_lsr(x, 11).to(torch.float64) + 1.0) * 2.0 ** -53
        del x
        r = torch.sqrt(-2.0 * torch.log(u[0::2]))
        th = (2.0 * math.pi) * u[1::2]
        z = torch.stack((r * torch.cos(th), r * torch.sin(th)), dim=1).reshape(-1)
        lo = 2 * p0
        hi = min(numel, lo + 2 * m)
        zc = z[: hi - lo]
        out[lo:hi] = zc if dtype == torch.float64 else zc.to(torch.float32).to(dtype)
    return out


# ---------------------------------------------------------------------------
# value distributions of the workloads
# ---------------------------------------------------------------------------

def softplus(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def log_decay(seed: int, stream: int, shape) -> np.ndarray:
    """g = -softplus(randn), stored as fp32 (alpha = exp(g) lies in (0, 1))."""
    return (-softplus(normal(seed, stream, shape))).astype(np.float32)


def beta_gate(seed: int, stream: int, shape) -> np.ndarray:
    """beta = sigmoid(randn), stored as fp32."""
    return sigmoid(normal(seed, stream, shape)).astype(np.float32)


def log_decay_torch(seed: int, stream: int, numel: int, device="cpu") -> torch.Tensor:
    """Flat fp32 tensor of g = -softplus(randn) (torch path, same definition)."""
    z = normal_torch(seed, stream, numel, device, torch.float64)
    return (-torch.nn.functional.softplus(z)).to(torch.float32)


def beta_gate_torch(seed: int, stream: int, numel: int, device="cpu") -> torch.Tensor:
    """Flat fp32 tensor of beta = sigmoid(randn) (torch path)."""
    return torch.sigmoid(normal_torch(seed, stream, numel, device, torch.float64)).to(torch.float32)


def slot_permutation(seed: int, stream: int, P: int) -> np.ndarray:
    """Seeded Fisher-Yates shuffle of the usable slots 1..P (row 0 is the
    padding row and never handed out)."""
    a = np.arange(1, P + 1, dtype=np.int32)
    if P > 1:
        u = uniform(seed, stream, P - 1)
        for n, i in enumerate(range(P - 1, 0, -1)):
            j = min(int(u[n] * (i + 1)), i)
            a[i], a[j] = a[j], a[i]
    return a


def to_torch(a: np.ndarray, dtype: str, device="cpu") -> torch.Tensor:
    """fp64/fp32 numpy -> torch tensor of storage dtype 'fp32' or 'bf16'
    (fp64 -> fp32 -> bf16, each nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)


TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeShape:
    """One decode layer: B requests, H_qk q/k heads, H_v value/state heads,
    head dims d_k/d_v, P usable pool slots (pool has P+1 rows)."""
    B: int
    Hqk: int
    Hv: int
    dk: int
    dv: int
    P: int
    kda: bool = True
    io: str = "bf16"
    state: str = "bf16"
    conv: str = "bf16"

    @property
    def C(self) -> int:
        return 2 * self.Hqk * self.dk + self.Hv * self.dv


def decode_inputs(sh: DecodeShape, seed: int, device="cpu", *, zero_state=False,
                  conv_w_scale: float = 0.5) -> dict:
    """Inputs of one decode step, drawn in the fixed stream order
    x, w, g, beta, conv state, ssm state, slots.  Returns torch tensors on
    ``device``: x [B,C] io; w [C,4] fp32; g [B,Hv,dk] or [B,Hv] fp32;
    beta [B,Hv] fp32; conv_pool [P+1,3,C]; ssm_pool [P+1,Hv,dv,dk]; slots [B]
    int32 (distinct, from 1..P)."""
    B, C = sh.B, sh.C
    x = to_torch(normal(seed, S_X, (B, C)), sh.io, device)
    w = to_torch(conv_w_scale * normal(seed, S_W, (C, 4)), "fp32", device)
    gshape = (B, sh.Hv, sh.dk) if sh.kda else (B, sh.Hv)
    g = torch.from_numpy(log_decay(seed, S_G, gshape)).to(device)
    beta = torch.from_numpy(beta_gate(seed, S_BETA, (B, sh.Hv))).to(device)
    dev_gen = device if torch.device(device).type != "cpu" else "cpu"
    n_conv = (sh.P + 1) * 3 * C
    n_ssm = (sh.P + 1) * sh.Hv * sh.dv * sh.dk
    if zero_state:
        conv_pool = torch.zeros(n_conv, dtype=TORCH_DTYPE[sh.conv], device=device)
        ssm_pool = torch.zeros(n_ssm, dtype=TORCH_DTYPE[sh.state], device=device)
    else:
        conv_pool = normal_torch(seed, S_CONV, n_conv, dev_gen, TORCH_DTYPE[sh.conv])
        ssm_pool = normal_torch(seed, S_SSM, n_ssm, dev_gen, TORCH_DTYPE[sh.state])
    slots = torch.from_numpy(slot_permutation(seed, S_SLOTS, sh.P)[:B].copy()).to(device)
    return dict(x=x, w=w, g=g, beta=beta,
                conv_pool=conv_pool.view(sh.P + 1, 3, C),
                ssm_pool=ssm_pool.view(sh.P + 1, sh.Hv, sh.dv, sh.dk),
                slots=slots)


@dataclass(frozen=True)
class PrefillShape:
    """Packed varlen prefill: sequence lengths, heads and dims."""
    seqlens: tuple
    Hqk: int
    Hv: int
    dk: int
    dv: int
    kda: bool = True
    io: str = "bf16"
    state: str = "fp32"

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))


def cu_seqlens(seqlens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))]).astype(np.int32)


def prefill_inputs(sh: PrefillShape, seed: int, device="cpu") -> dict:
    """q, k [T,Hqk,dk], v [T,Hv,dv] (io dtype, randn); g [T,Hv,dk] or [T,Hv]
    (-softplus(randn), fp32); beta [T,Hv] (sigmoid(randn), fp32);
    cu_seqlens [N+1] int32."""
    T = sh.T
    dev_gen = device if torch.device(device).type != "cpu" else "cpu"
    q = normal_torch(seed, S_Q, T * sh.Hqk * sh.dk, dev_gen, TORCH_DTYPE[sh.io])
    k = normal_torch(seed, S_K, T * sh.Hqk * sh.dk, dev_gen, TORCH_DTYPE[sh.io])
    v = normal_torch(seed, S_V, T * sh.Hv * sh.dv, dev_gen, TORCH_DTYPE[sh.io])
    gshape = (T, sh.Hv, sh.dk) if sh.kda else (T, sh.Hv)
    g = torch.from_numpy(log_decay(seed, S_G, gshape)).to(device)
    beta = torch.from_numpy(beta_gate(seed, S_BETA, (T, sh.Hv))).to(device)
    cu = torch.from_numpy(cu_seqlens(sh.seqlens)).to(device)
    return dict(q=q.view(T, sh.Hqk, sh.dk), k=k.view(T, sh.Hqk, sh.dk),
                v=v.view(T, sh.Hv, sh.dv), g=g, beta=beta, cu_seqlens=cu)
