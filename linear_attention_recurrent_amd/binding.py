"""ctypes binding of ``libla.so`` (the C ABI in ``include/la.h``).

Argument marshalling only: shapes, dtypes and strides are read off torch
tensors, raw device pointers and the current HIP stream are passed through,
and a non-zero status is raised as :class:`LAError` with the library's
message.  Every step of the computation runs in the HIP kernels; if the
library is missing, loading it raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libla.so")
_lib = None

LA_F32, LA_BF16 = 0, 1
LA_PREFILL_FP32, LA_PREFILL_BF16X3 = 0, 1
_DT = {torch.float32: LA_F32, torch.bfloat16: LA_BF16}
_DT_NAME = {"fp32": LA_F32, "bf16": LA_BF16}


class LAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libla status {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


class LaRing(ctypes.Structure):
    """``la_ring`` of include/la.h (device pointers of the ring arrays)."""
    _fields_ = [("L", ctypes.c_int), ("d", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("rawv", ctypes.c_void_p), ("rawk", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("beta", ctypes.c_void_p)]


def load_library():
    """Load ``libla.so`` (built by ``linear_attention_recurrent_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python -m "
                          "linear_attention_recurrent_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, L, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "la_version": ([], I),
        "la_last_error": ([], ctypes.c_char_p),
        "la_pool_bytes": ([I, I, I, I, I, I, I, I, P, P], I),
        "shortconv_update": ([I, I, P, I, P, P, P, L, I, I, P, P, P], I),
        "kda_decode_step": ([I, I, I, I, I, P, I, P, P, P, L, I, P, P, P, I, P, L, I, P, F, F, P], I),
        "gdn_decode_step": ([I, I, I, I, I, P, I, P, P, P, L, I, P, P, P, I, P, L, I, P, F, F, P], I),
        "shortconv_prefill": ([I, I, I, P, I, P, P, P, P, P, P, L, I, I, P, P], I),
        "kda_prefill_chunked": ([I, I, I, I, I, I, P, L, P, L, P, L, I, P, P, P, P, P, I, P, L, I,
                                 P, F, F, I, P, Z, P], I),
        "gdn_prefill_chunked": ([I, I, I, I, I, I, P, L, P, L, P, L, I, P, P, P, P, P, I, P, L, I,
                                 P, F, F, I, P, Z, P], I),
        "kda_prefill_conv": ([I, I, I, I, I, I, P, I, P, P, P, L, I, P, P, P, P, P, I, P, L, I,
                              P, F, F, I, P, Z, P], I),
        "gdn_prefill_conv": ([I, I, I, I, I, I, P, I, P, P, P, L, I, P, P, P, P, P, I, P, L, I,
                              P, F, F, I, P, Z, P], I),
        "kda_prefill_chunked_noalloc": ([I, I, I, I, I, I, P, L, P, L, P, L, I, P, P, P, P, P, I,
                                         P, L, I, P, F, F, I, P], I),
        "kda_prefill_workspace_bytes": ([I, I, I, I, I, I, I], Z),
        "gdn_prefill_workspace_bytes": ([I, I, I, I, I, I, I], Z),
        "la_ring_bytes": ([I, I, I, I, I, I, I, I, P, P, P, P], I),
        "kda_verify": ([I, I, P, I, I, I, I, P, I, P, P, P, L, I, P, P, P, I, P, L, I, P, P,
                        ctypes.POINTER(LaRing), P, F, F, P], I),
        "gdn_verify": ([I, I, P, I, I, I, I, P, I, P, P, P, L, I, P, P, P, I, P, L, I, P, P,
                        ctypes.POINTER(LaRing), P, F, F, P], I),
        "kda_commit": ([I, P, I, I, I, P, I, P, L, I, I, ctypes.POINTER(LaRing), P, F, P], I),
        "gdn_commit": ([I, P, I, I, I, P, I, P, L, I, I, ctypes.POINTER(LaRing), P, F, P], I),
        "conv_window_scatter": ([I, I, I, P, P, P, P, P, L, I, I, P], I),
        "kda_ring_fold": ([I, P, I, I, I, P, P, I, P, L, I, I, ctypes.POINTER(LaRing), P, P, P, F,
                           F, P], I),
        "gdn_ring_fold": ([I, P, I, I, I, P, P, I, P, L, I, I, ctypes.POINTER(LaRing), P, P, P, F,
                           F, P], I),
        "state_track_copy": ([I, P, P, P, P, L, L, I, P, L, L, I, I, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise LAError(rc, load_library().la_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype} (fp32 or bf16)")
    return _DT[t.dtype]


# ---- argument checks (before any launch: a wrong dtype, length or device
#      would otherwise make a kernel read past an allocation) ----

F32, I32 = torch.float32, torch.int32
_FLOATS = (torch.float32, torch.bfloat16)


def _arg(t, what, *, dtype=None, shape=None, contig=True):
    """Checks a tensor argument's dtype (one dtype or a tuple), exact shape
    and contiguity; returns it."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor, got {type(t).__name__}")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contig and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _opt(t, what, **kw):
    return None if t is None else _arg(t, what, **kw)


def _devices(ref: torch.Tensor, **named):
    """Every named tensor (None skipped) must sit on ref's GPU."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU (got {ref.device})")
    for what, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{what} is on {t.device}, the pools on {ref.device}")


def _row_view(pool: torch.Tensor, inner: tuple, what: str) -> int:
    """Checks a pool [rows, *inner] has contiguous inner dims; returns the row
    stride in elements."""
    if not isinstance(pool, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if pool.dtype not in _FLOATS:
        raise ValueError(f"{what}: dtype {pool.dtype}, expected fp32 or bf16")
    if tuple(pool.shape[1:]) != tuple(inner):
        raise ValueError(f"{what}: expected rows of shape {inner}, got {tuple(pool.shape[1:])}")
    if not pool[0].is_contiguous():
        raise ValueError(f"{what}: inner dims must be contiguous")
    return pool.stride(0)


def _contig(t: torch.Tensor, what: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def version() -> int:
    return load_library().la_version()


def pool_bytes(layers: int, slots: int, Hv: int, dv: int, dk: int, conv_channels: int,
               state_dtype: str = "bf16", conv_dtype: str = "bf16"):
    """(ssm_bytes, conv_bytes) of per-layer pools with slots + 1 rows."""
    s, c = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().la_pool_bytes(layers, slots, Hv, dv, dk, conv_channels,
                                        _DT_NAME[state_dtype], _DT_NAME[conv_dtype],
                                        ctypes.byref(s), ctypes.byref(c)))
    return s.value, c.value


def ring_bytes(layers: int, slots: int, Hv: int, L: int, dk: int, dv: int,
               io_dtype: str = "bf16", kda: bool = True) -> dict:
    """Bytes of each ReplaySSM ring buffer (slots + 1 rows): d, k, rawv, rawk,
    g, beta."""
    d, k, g, b = (ctypes.c_int64() for _ in range(4))
    _check(load_library().la_ring_bytes(layers, slots, Hv, L, dk, dv, _DT_NAME[io_dtype],
                                        int(kda), ctypes.byref(d), ctypes.byref(k),
                                        ctypes.byref(g), ctypes.byref(b)))
    return {"d": d.value, "k": k.value, "rawv": d.value, "rawk": k.value, "g": g.value,
            "beta": b.value}


def shortconv_update(x, w, conv_pool, slots, bias=None, y=None):
    """One decode token of the short conv + SiLU; rolls conv_pool rows in place.
    x [B, C]; w [C, 4] fp32; conv_pool [P+1, 3, C]; slots [B] int32."""
    _arg(x, "x", dtype=_FLOATS)
    if x.dim() != 2:
        raise ValueError(f"x: expected [B, C], got {tuple(x.shape)}")
    B, C = x.shape
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    _arg(w, "w", dtype=F32, shape=(C, 4))
    _opt(bias, "bias", dtype=F32, shape=(C,))
    _arg(slots, "slots", dtype=I32, shape=(B,))
    _opt(y, "y", dtype=x.dtype, shape=(B, C))
    _devices(conv_pool, x=x, w=w, bias=bias, slots=slots, y=y)
    y = torch.empty_like(x) if y is None else y
    _check(load_library().shortconv_update(
        B, C, _ptr(x), _dtype(x), _ptr(w), _ptr(bias), _ptr(conv_pool), stride,
        _dtype(conv_pool), conv_pool.shape[0], _ptr(slots), _ptr(y), _stream(x.device)))
    return y


def _decode(kda, x, g, beta, slots, ssm_pool, *, Hqk, conv_w=None, conv_b=None,
            conv_pool=None, out=None, eps=1e-6, scale=1.0):
    _arg(x, "x", dtype=_FLOATS)
    if x.dim() != 2:
        raise ValueError(f"x: expected [B, C], got {tuple(x.shape)}")
    B, C = x.shape
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(g, "g", dtype=F32, shape=(B, Hv, dk) if kda else (B, Hv))
    _arg(beta, "beta", dtype=F32, shape=(B, Hv))
    _arg(slots, "slots", dtype=I32, shape=(B,))
    _opt(out, "out", dtype=x.dtype, shape=(B, Hv, dv))
    cstride, cdt = 0, LA_F32
    if conv_w is not None:
        if conv_pool is None:
            raise ValueError("conv_pool is required with conv_w")
        cstride = _row_view(conv_pool, (3, C), "conv_pool")
        cdt = _dtype(conv_pool)
        _arg(conv_w, "conv_w", dtype=F32, shape=(C, 4))
        _opt(conv_b, "conv_b", dtype=F32, shape=(C,))
    _devices(ssm_pool, x=x, g=g, beta=beta, slots=slots, out=out, conv_w=conv_w, conv_b=conv_b,
             conv_pool=conv_pool)
    out = torch.empty((B, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    fn = load_library().kda_decode_step if kda else load_library().gdn_decode_step
    _check(fn(B, Hqk, Hv, dk, dv, _ptr(x), _dtype(x), _ptr(conv_w), _ptr(conv_b),
              _ptr(conv_pool), cstride, cdt, _ptr(g), _ptr(beta), _ptr(slots), rows,
              _ptr(ssm_pool), sstride, _dtype(ssm_pool), _ptr(out), eps, scale,
              _stream(x.device)))
    return out


def kda_decode_step(x, g, beta, slots, ssm_pool, *, Hqk, conv_w=None, conv_b=None,
                    conv_pool=None, out=None, eps=1e-6, scale=1.0):
    """Fused KDA decode.  x [B, C]; g [B, Hv, dk] fp32; beta [B, Hv] fp32;
    slots [B] int32; ssm_pool [P+1, Hv, dv, dk] (a row view of a larger pool
    is fine); conv_w [C, 4] (None: x is post-conv); conv_pool [P+1, 3, C].
    Returns out [B, Hv, dv] (x's dtype)."""
    return _decode(True, x, g, beta, slots, ssm_pool, Hqk=Hqk, conv_w=conv_w, conv_b=conv_b,
                   conv_pool=conv_pool, out=out, eps=eps, scale=scale)


def gdn_decode_step(x, g, beta, slots, ssm_pool, *, Hqk, conv_w=None, conv_b=None,
                    conv_pool=None, out=None, eps=1e-6, scale=1.0):
    """Fused GDN decode; as :func:`kda_decode_step` with g [B, Hv]."""
    return _decode(False, x, g, beta, slots, ssm_pool, Hqk=Hqk, conv_w=conv_w, conv_b=conv_b,
                   conv_pool=conv_pool, out=out, eps=eps, scale=scale)


def _seq_args(cu_seqlens, slot_in, slot_out):
    """cu_seqlens [N+1], slot_in / slot_out [N], all int32; returns N."""
    _arg(cu_seqlens, "cu_seqlens", dtype=I32)
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens: expected [N+1]")
    N = cu_seqlens.shape[0] - 1
    _arg(slot_in, "slot_in", dtype=I32, shape=(N,))
    _arg(slot_out, "slot_out", dtype=I32, shape=(N,))
    return N


def shortconv_prefill(x, cu_seqlens, slot_in, slot_out, w, conv_pool, bias=None, y=None):
    """Short conv + SiLU over packed sequences.  x [T, C]; cu_seqlens [N+1];
    slot_in/slot_out [N] int32; conv_pool [P+1, 3, C].  Returns y [T, C]."""
    _arg(x, "x", dtype=_FLOATS)
    if x.dim() != 2:
        raise ValueError(f"x: expected [T, C], got {tuple(x.shape)}")
    T, C = x.shape
    N = _seq_args(cu_seqlens, slot_in, slot_out)
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    _arg(w, "w", dtype=F32, shape=(C, 4))
    _opt(bias, "bias", dtype=F32, shape=(C,))
    _opt(y, "y", dtype=x.dtype, shape=(T, C))
    _devices(conv_pool, x=x, cu_seqlens=cu_seqlens, slot_in=slot_in, slot_out=slot_out, w=w,
             bias=bias, y=y)
    y = torch.empty_like(x) if y is None else y
    _check(load_library().shortconv_prefill(
        N, T, C, _ptr(x), _dtype(x), _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out), _ptr(w),
        _ptr(bias), _ptr(conv_pool), stride, _dtype(conv_pool), conv_pool.shape[0], _ptr(y),
        _stream(x.device)))
    return y


def kda_prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode=LA_PREFILL_FP32) -> int:
    return load_library().kda_prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode)


def gdn_prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode=LA_PREFILL_FP32) -> int:
    return load_library().gdn_prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode)


def prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode=LA_PREFILL_FP32, kda=True) -> int:
    """Workspace bytes of the KDA (kda=True) or GDN prefill calls."""
    fn = kda_prefill_workspace_bytes if kda else gdn_prefill_workspace_bytes
    return fn(N, T, Hqk, Hv, dk, dv, mode)


def _token_view(t, T, heads, d, dtype, what):
    _arg(t, what, dtype=dtype, contig=False)
    if t.dim() != 3 or tuple(t.shape) != (T, heads, d):
        raise ValueError(f"{what}: expected [{T}, {heads}, {d}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError(f"{what}: heads and channels must be contiguous inside a token")
    return t.stride(0)


def _workspace(workspace, need, dev):
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    _arg(workspace, "workspace")
    if workspace.device != dev:
        raise ValueError(f"workspace is on {workspace.device}, the pools on {dev}")
    return workspace


def _prefill(kda, q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, *, out=None,
             eps=1e-6, scale=1.0, mode=LA_PREFILL_FP32, workspace=None):
    _arg(q, "q", dtype=_FLOATS, contig=False)
    if q.dim() != 3:
        raise ValueError(f"q: expected [T, Hqk, dk], got {tuple(q.shape)}")
    T, Hqk, dk = q.shape
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, _ = ssm_pool.shape
    N = _seq_args(cu_seqlens, slot_in, slot_out)
    qs = _token_view(q, T, Hqk, dk, q.dtype, "q")
    ks = _token_view(k, T, Hqk, dk, q.dtype, "k")
    vs = _token_view(v, T, Hv, dv, q.dtype, "v")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(g, "g", dtype=F32, shape=(T, Hv, dk) if kda else (T, Hv))
    _arg(beta, "beta", dtype=F32, shape=(T, Hv))
    _opt(out, "out", dtype=q.dtype, shape=(T, Hv, dv))
    _devices(ssm_pool, q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, slot_in=slot_in,
             slot_out=slot_out, out=out)
    out = torch.empty((T, Hv, dv), dtype=q.dtype, device=q.device) if out is None else out
    workspace = _workspace(workspace, prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode, kda),
                           ssm_pool.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load_library().kda_prefill_chunked if kda else load_library().gdn_prefill_chunked
    _check(fn(N, T, Hqk, Hv, dk, dv, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dtype(q),
              _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out), rows,
              _ptr(ssm_pool), sstride, _dtype(ssm_pool), _ptr(out), eps, scale, mode,
              _ptr(workspace), ws_bytes, _stream(q.device)))
    return out


def kda_prefill_chunked_noalloc(q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, *,
                                out, eps=1e-6, scale=1.0, mode=LA_PREFILL_FP32):
    """kda_prefill_chunked with the library's own 128 MiB per-GPU scratch in
    place of a workspace: the call allocates nothing (``out`` [T, Hv, dv] is
    the caller's).  Calls that overlap on one GPU race."""
    _arg(q, "q", dtype=_FLOATS, contig=False)
    if q.dim() != 3:
        raise ValueError(f"q: expected [T, Hqk, dk], got {tuple(q.shape)}")
    T, Hqk, dk = q.shape
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, _ = ssm_pool.shape
    N = _seq_args(cu_seqlens, slot_in, slot_out)
    qs = _token_view(q, T, Hqk, dk, q.dtype, "q")
    ks = _token_view(k, T, Hqk, dk, q.dtype, "k")
    vs = _token_view(v, T, Hv, dv, q.dtype, "v")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(g, "g", dtype=F32, shape=(T, Hv, dk))
    _arg(beta, "beta", dtype=F32, shape=(T, Hv))
    _arg(out, "out", dtype=q.dtype, shape=(T, Hv, dv))
    _devices(ssm_pool, q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu_seqlens, slot_in=slot_in,
             slot_out=slot_out, out=out)
    _check(load_library().kda_prefill_chunked_noalloc(
        N, T, Hqk, Hv, dk, dv, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dtype(q), _ptr(g),
        _ptr(beta), _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out), rows, _ptr(ssm_pool),
        sstride, _dtype(ssm_pool), _ptr(out), eps, scale, mode, _stream(q.device)))
    return out


def kda_prefill_chunked(q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw):
    """Chunked KDA prefill.  q, k [T, Hqk, dk], v [T, Hv, dv] (token-strided
    views are fine); g [T, Hv, dk]; beta [T, Hv]; cu_seqlens [N+1]; slot_in,
    slot_out [N]; ssm_pool [P+1, Hv, dv, dk].  Returns out [T, Hv, dv]."""
    return _prefill(True, q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw)


def gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw):
    """Chunked GDN prefill; as :func:`kda_prefill_chunked` with g [T, Hv]."""
    return _prefill(False, q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw)


def _prefill_conv(kda, x, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, *, Hqk, conv_w,
                  conv_pool, conv_b=None, out=None, eps=1e-6, scale=1.0, mode=LA_PREFILL_FP32,
                  workspace=None):
    _arg(x, "x", dtype=_FLOATS)
    if x.dim() != 2:
        raise ValueError(f"x: expected [T, C], got {tuple(x.shape)}")
    T, C = x.shape
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    N = _seq_args(cu_seqlens, slot_in, slot_out)
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    cstride = _row_view(conv_pool, (3, C), "conv_pool")
    _arg(conv_w, "conv_w", dtype=F32, shape=(C, 4))
    _opt(conv_b, "conv_b", dtype=F32, shape=(C,))
    _arg(g, "g", dtype=F32, shape=(T, Hv, dk) if kda else (T, Hv))
    _arg(beta, "beta", dtype=F32, shape=(T, Hv))
    _opt(out, "out", dtype=x.dtype, shape=(T, Hv, dv))
    _devices(ssm_pool, x=x, g=g, beta=beta, cu_seqlens=cu_seqlens, slot_in=slot_in,
             slot_out=slot_out, conv_w=conv_w, conv_b=conv_b, conv_pool=conv_pool, out=out)
    out = torch.empty((T, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    workspace = _workspace(workspace, prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode, kda),
                           ssm_pool.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load_library().kda_prefill_conv if kda else load_library().gdn_prefill_conv
    _check(fn(N, T, Hqk, Hv, dk, dv, _ptr(x), _dtype(x), _ptr(conv_w), _ptr(conv_b),
              _ptr(conv_pool), cstride, _dtype(conv_pool), _ptr(g), _ptr(beta),
              _ptr(cu_seqlens), _ptr(slot_in), _ptr(slot_out), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _ptr(out), eps, scale, mode, _ptr(workspace), ws_bytes,
              _stream(x.device)))
    return out


def kda_prefill_conv(x, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw):
    """Chunked KDA prefill with the short conv fused into its loads.
    x [T, C] pre-conv q|k|v projections; conv_w [C, 4]; conv_b [C] or None;
    conv_pool [P+1, 3, C] (same slots as ssm_pool); Hqk keyword; the rest as
    :func:`kda_prefill_chunked`.  Returns out [T, Hv, dv]."""
    return _prefill_conv(True, x, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw)


def gdn_prefill_conv(x, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw):
    """GDN form of :func:`kda_prefill_conv` (g [T, Hv])."""
    return _prefill_conv(False, x, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, **kw)


# ------------------------------------------------------ speculative decode --

def new_ring(num_rows, Hv, L, dk, dv, *, kda=True, dtype=torch.bfloat16, device="cuda"):
    """Allocates a zeroed ReplaySSM ring (dict of tensors) for a pool of
    num_rows rows: d, rawv [rows, Hv, L, dv] and k, rawk [rows, Hv, L, dk] in
    `dtype` (the I/O dtype of the verify calls), g [rows, Hv, L, dk] (KDA) or
    [rows, Hv, L] (GDN) and beta [rows, Hv, L] in fp32."""
    z = lambda *sh, dt=dtype: torch.zeros(sh, dtype=dt, device=device)  # noqa: E731
    return {"d": z(num_rows, Hv, L, dv), "k": z(num_rows, Hv, L, dk),
            "rawv": z(num_rows, Hv, L, dv), "rawk": z(num_rows, Hv, L, dk),
            "g": z(*((num_rows, Hv, L, dk) if kda else (num_rows, Hv, L)), dt=torch.float32),
            "beta": z(num_rows, Hv, L, dt=torch.float32)}


def _ring_struct(ring, rows, Hv, dk, dv, kda, io_dtype, ref):
    """Checks the ring's buffers against the pool (rows, heads, dims), the
    I/O dtype and the device; returns the la_ring struct."""
    d = _arg(ring["d"], "ring['d']", dtype=io_dtype)
    if d.dim() != 4:
        raise ValueError("ring['d']: expected [rows, Hv, L, dv]")
    L = d.shape[2]
    _arg(d, "ring['d']", shape=(rows, Hv, L, dv))
    _arg(ring["rawv"], "ring['rawv']", dtype=io_dtype, shape=(rows, Hv, L, dv))
    _arg(ring["k"], "ring['k']", dtype=io_dtype, shape=(rows, Hv, L, dk))
    _arg(ring["rawk"], "ring['rawk']", dtype=io_dtype, shape=(rows, Hv, L, dk))
    _arg(ring["g"], "ring['g']", dtype=F32, shape=(rows, Hv, L, dk) if kda else (rows, Hv, L))
    _arg(ring["beta"], "ring['beta']", dtype=F32, shape=(rows, Hv, L))
    _devices(ref, **{f"ring[{k!r}]": ring[k] for k in ("d", "k", "rawv", "rawk", "g", "beta")})
    return LaRing(L, ring["d"].data_ptr(), ring["k"].data_ptr(), ring["rawv"].data_ptr(),
                  ring["rawk"].data_ptr(), ring["g"].data_ptr(), ring["beta"].data_ptr())


def _verify(kda, x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, *, Hqk, conv_w=None,
            conv_b=None, conv_pool=None, out=None, windows=None, eps=1e-6, scale=1.0):
    _arg(x, "x", dtype=_FLOATS)
    if x.dim() != 3:
        raise ValueError(f"x: expected [B, D, C], got {tuple(x.shape)}")
    B, D, C = x.shape
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(g, "g", dtype=F32, shape=(B, D, Hv, dk) if kda else (B, D, Hv))
    _arg(beta, "beta", dtype=F32, shape=(B, D, Hv))
    _arg(slots, "slots", dtype=I32, shape=(B,))
    _arg(n_tok, "n_tok", dtype=I32, shape=(B,))
    _arg(ring_base, "ring_base", dtype=I32, shape=(B,))
    _opt(out, "out", dtype=x.dtype, shape=(B, D, Hv, dv))
    cstride, cdt = 0, LA_F32
    if conv_w is not None:
        if conv_pool is None:
            raise ValueError("conv_pool is required with conv_w")
        cstride = _row_view(conv_pool, (3, C), "conv_pool")
        cdt = _dtype(conv_pool)
        _arg(conv_w, "conv_w", dtype=F32, shape=(C, 4))
        _opt(conv_b, "conv_b", dtype=F32, shape=(C,))
        _opt(windows, "windows", dtype=conv_pool.dtype, shape=(B, D, 3, C))
    r = _ring_struct(ring, rows, Hv, dk, dv, kda, x.dtype, ssm_pool)
    _devices(ssm_pool, x=x, g=g, beta=beta, slots=slots, n_tok=n_tok, ring_base=ring_base,
             out=out, conv_w=conv_w, conv_b=conv_b, conv_pool=conv_pool, windows=windows)
    if conv_w is not None and windows is None:
        windows = torch.empty((B, D, 3, C), dtype=conv_pool.dtype, device=x.device)
    out = torch.empty((B, D, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    fn = load_library().kda_verify if kda else load_library().gdn_verify
    _check(fn(B, D, _ptr(n_tok), Hqk, Hv, dk, dv, _ptr(x), _dtype(x), _ptr(conv_w),
              _ptr(conv_b), _ptr(conv_pool), cstride, cdt, _ptr(g), _ptr(beta), _ptr(slots),
              rows, _ptr(ssm_pool), sstride, _dtype(ssm_pool), _ptr(out), _ptr(windows),
              ctypes.byref(r), _ptr(ring_base), eps, scale, _stream(x.device)))
    return out, windows


def kda_verify(x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, **kw):
    """KDA speculative verify of D draft tokens per request.  x [B, D, C];
    g [B, D, Hv, dk]; beta [B, D, Hv]; slots, n_tok, ring_base [B] int32;
    ring from :func:`new_ring`.  The pools are not modified.  Returns
    (out [B, D, Hv, dv], conv windows [B, D, 3, C] or None)."""
    return _verify(True, x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, **kw)


def gdn_verify(x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, **kw):
    """GDN verify; as :func:`kda_verify` with g [B, D, Hv]."""
    return _verify(False, x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, **kw)


def _commit(kda, accepted, slots, ssm_pool, ring, ring_base, eps=1e-6):
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, dk = ssm_pool.shape
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(slots, "slots", dtype=I32)
    if slots.dim() != 1:
        raise ValueError("slots: expected [B]")
    B = slots.shape[0]
    _arg(accepted, "accepted", dtype=I32, shape=(B,))
    _arg(ring_base, "ring_base", dtype=I32, shape=(B,))
    io = ring["d"].dtype
    if io not in _FLOATS:
        raise ValueError(f"ring['d']: dtype {io}, expected fp32 or bf16")
    r = _ring_struct(ring, rows, Hv, dk, dv, kda, io, ssm_pool)
    _devices(ssm_pool, accepted=accepted, slots=slots, ring_base=ring_base)
    fn = load_library().kda_commit if kda else load_library().gdn_commit
    _check(fn(B, _ptr(accepted), Hv, dk, dv, _ptr(slots), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _DT[io], ctypes.byref(r), _ptr(ring_base), eps,
              _stream(ssm_pool.device)))


def kda_commit(accepted, slots, ssm_pool, ring, ring_base, eps=1e-6):
    """Exact commit: replays the first accepted[b] ring steps of each request
    from its pool row, in place."""
    _commit(True, accepted, slots, ssm_pool, ring, ring_base, eps)


def gdn_commit(accepted, slots, ssm_pool, ring, ring_base, eps=1e-6):
    """GDN exact commit; as :func:`kda_commit`."""
    _commit(False, accepted, slots, ssm_pool, ring, ring_base, eps)


def _mask(mask, B):
    if mask is None:
        return None
    if mask.dtype not in (torch.uint8, torch.bool):
        raise ValueError(f"mask: dtype {mask.dtype}, expected uint8 or bool")
    return _arg(mask.to(torch.uint8), "mask", shape=(B,))


def conv_window_scatter(windows, slots, step, conv_pool, mask=None):
    """conv_pool[slots[b]] = windows[b, step[b]] where mask[b] (uint8 or bool;
    None = all) and 0 <= step[b] < D."""
    _arg(windows, "windows", dtype=_FLOATS)
    if windows.dim() != 4 or windows.shape[2] != 3:
        raise ValueError(f"windows: expected [B, D, 3, C], got {tuple(windows.shape)}")
    B, D, _, C = windows.shape
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    if windows.dtype != conv_pool.dtype:
        raise ValueError("windows must have the conv pool's dtype")
    _arg(slots, "slots", dtype=I32, shape=(B,))
    _arg(step, "step", dtype=I32, shape=(B,))
    mask = _mask(mask, B)
    _devices(conv_pool, windows=windows, slots=slots, step=step, mask=mask)
    _check(load_library().conv_window_scatter(
        B, D, C, _ptr(mask), _ptr(slots), _ptr(step), _ptr(windows), _ptr(conv_pool), stride,
        _dtype(conv_pool), conv_pool.shape[0], _stream(conv_pool.device)))


def state_track_copy(src, dst, conv_pool, ssm_pool, mask=None):
    """Rows dst[b] of both pools become copies of rows src[b] where mask[b]."""
    for pool, what in ((conv_pool, "conv_pool"), (ssm_pool, "ssm_pool")):
        if not isinstance(pool, torch.Tensor) or pool.dtype not in _FLOATS:
            raise ValueError(f"{what}: expected an fp32 or bf16 tensor")
        if not pool[0].is_contiguous():
            raise ValueError("pool rows must be contiguous")
    if conv_pool.shape[0] != ssm_pool.shape[0]:
        raise ValueError("conv_pool and ssm_pool must have the same number of rows")
    _arg(src, "src", dtype=I32)
    if src.dim() != 1:
        raise ValueError("src: expected [B]")
    B = src.shape[0]
    _arg(dst, "dst", dtype=I32, shape=(B,))
    mask = _mask(mask, B)
    _devices(ssm_pool, conv_pool=conv_pool, src=src, dst=dst, mask=mask)
    crow = conv_pool[0].numel()
    srow = ssm_pool[0].numel()
    _check(load_library().state_track_copy(
        B, _ptr(mask), _ptr(src), _ptr(dst), _ptr(conv_pool), conv_pool.stride(0), crow,
        _dtype(conv_pool), _ptr(ssm_pool), ssm_pool.stride(0), srow, _dtype(ssm_pool),
        ssm_pool.shape[0], _stream(ssm_pool.device)))


def _fold(kda, m, slots, ssm_pool, ring, ring_base, dst=None, q=None, out=None, eps=1e-6,
          scale=1.0):
    if ssm_pool.dim() != 4:
        raise ValueError("ssm_pool: expected [P+1, Hv, dv, dk]")
    rows, Hv, dv, dk = ssm_pool.shape
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    _arg(slots, "slots", dtype=I32)
    if slots.dim() != 1:
        raise ValueError("slots: expected [B]")
    B = slots.shape[0]
    _arg(m, "m", dtype=I32, shape=(B,))
    _arg(ring_base, "ring_base", dtype=I32, shape=(B,))
    _opt(dst, "dst", dtype=I32, shape=(B,))
    io = ring["d"].dtype
    if io not in _FLOATS:
        raise ValueError(f"ring['d']: dtype {io}, expected fp32 or bf16")
    _opt(q, "q", dtype=io, shape=(B, Hv, dk))
    _opt(out, "out", dtype=io, shape=(B, Hv, dv))
    r = _ring_struct(ring, rows, Hv, dk, dv, kda, io, ssm_pool)
    _devices(ssm_pool, m=m, slots=slots, ring_base=ring_base, dst=dst, q=q, out=out)
    if q is not None and out is None:
        out = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    fn = load_library().kda_ring_fold if kda else load_library().gdn_ring_fold
    _check(fn(B, _ptr(m), Hv, dk, dv, _ptr(slots), _ptr(dst), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _DT[io], ctypes.byref(r), _ptr(ring_base), _ptr(q), _ptr(out),
              eps, scale, _stream(ssm_pool.device)))
    return out


def kda_ring_fold(m, slots, ssm_pool, ring, ring_base, dst=None, q=None, out=None, eps=1e-6,
                  scale=1.0):
    """ReplaySSM fast rebuild: folds m[b] ring steps (d, k, g) into the
    checkpoint rows slots[b], storing the state to rows dst[b] (None: in
    place); with q [B, Hv, dk] returns out = scale S_m q_hat."""
    return _fold(True, m, slots, ssm_pool, ring, ring_base, dst, q, out, eps, scale)


def gdn_ring_fold(m, slots, ssm_pool, ring, ring_base, dst=None, q=None, out=None, eps=1e-6,
                  scale=1.0):
    """GDN fast rebuild; as :func:`kda_ring_fold`."""
    return _fold(False, m, slots, ssm_pool, ring, ring_base, dst, q, out, eps, scale)
