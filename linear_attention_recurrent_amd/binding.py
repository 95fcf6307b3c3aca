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
        "prefill_workspace_bytes": ([I, I, I, I, I, I, I], Z),
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


def _row_view(pool: torch.Tensor, inner: tuple, what: str) -> int:
    """Checks a pool [rows, *inner] has contiguous inner dims; returns the row
    stride in elements."""
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


def shortconv_update(x, w, conv_pool, slots, bias=None, y=None):
    """One decode token of the short conv + SiLU; rolls conv_pool rows in place.
    x [B, C]; w [C, 4] fp32; conv_pool [P+1, 3, C]; slots [B] int32."""
    B, C = x.shape
    _contig(x, "x")
    y = torch.empty_like(x) if y is None else y
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    _check(load_library().shortconv_update(
        B, C, _ptr(x), _dtype(x), _ptr(_contig(w, "w")), _ptr(bias), _ptr(conv_pool), stride,
        _dtype(conv_pool), conv_pool.shape[0], _ptr(_contig(slots, "slots")), _ptr(y),
        _stream(x.device)))
    return y


def _decode(kda, x, g, beta, slots, ssm_pool, *, Hqk, conv_w=None, conv_b=None,
            conv_pool=None, out=None, eps=1e-6, scale=1.0):
    B, C = x.shape
    _contig(x, "x")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    cstride, cdt = 0, LA_F32
    if conv_w is not None:
        cstride = _row_view(conv_pool, (3, C), "conv_pool")
        cdt = _dtype(conv_pool)
    out = torch.empty((B, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    fn = load_library().kda_decode_step if kda else load_library().gdn_decode_step
    _check(fn(B, Hqk, Hv, dk, dv, _ptr(x), _dtype(x), _ptr(conv_w), _ptr(conv_b),
              _ptr(conv_pool), cstride, cdt, _ptr(_contig(g, "g")), _ptr(_contig(beta, "beta")),
              _ptr(_contig(slots, "slots")), rows, _ptr(ssm_pool), sstride, _dtype(ssm_pool),
              _ptr(_contig(out, "out")), eps, scale, _stream(x.device)))
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


def shortconv_prefill(x, cu_seqlens, slot_in, slot_out, w, conv_pool, bias=None, y=None):
    """Short conv + SiLU over packed sequences.  x [T, C]; cu_seqlens [N+1];
    slot_in/slot_out [N] int32; conv_pool [P+1, 3, C].  Returns y [T, C]."""
    T, C = x.shape
    _contig(x, "x")
    N = cu_seqlens.shape[0] - 1
    y = torch.empty_like(x) if y is None else y
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    _check(load_library().shortconv_prefill(
        N, T, C, _ptr(x), _dtype(x), _ptr(_contig(cu_seqlens, "cu_seqlens")),
        _ptr(_contig(slot_in, "slot_in")), _ptr(_contig(slot_out, "slot_out")),
        _ptr(_contig(w, "w")), _ptr(bias), _ptr(conv_pool), stride, _dtype(conv_pool),
        conv_pool.shape[0], _ptr(y), _stream(x.device)))
    return y


def prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode=LA_PREFILL_FP32) -> int:
    return load_library().prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode)


def _token_view(t, heads, d, what):
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != d:
        raise ValueError(f"{what}: expected [T, {heads}, {d}]")
    if t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError(f"{what}: heads and channels must be contiguous inside a token")
    return t.stride(0)


def _prefill(kda, q, k, v, g, beta, cu_seqlens, slot_in, slot_out, ssm_pool, *, out=None,
             eps=1e-6, scale=1.0, mode=LA_PREFILL_FP32, workspace=None):
    T, Hqk, dk = q.shape
    rows, Hv, dv, _ = ssm_pool.shape
    N = cu_seqlens.shape[0] - 1
    qs = _token_view(q, Hqk, dk, "q")
    ks = _token_view(k, Hqk, dk, "k")
    vs = _token_view(v, Hv, dv, "v")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    out = torch.empty((T, Hv, dv), dtype=q.dtype, device=q.device) if out is None else out
    need = prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load_library().kda_prefill_chunked if kda else load_library().gdn_prefill_chunked
    _check(fn(N, T, Hqk, Hv, dk, dv, _ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _dtype(q),
              _ptr(_contig(g, "g")), _ptr(_contig(beta, "beta")),
              _ptr(_contig(cu_seqlens, "cu_seqlens")), _ptr(_contig(slot_in, "slot_in")),
              _ptr(_contig(slot_out, "slot_out")), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _ptr(_contig(out, "out")), eps, scale, mode, _ptr(workspace),
              ws_bytes, _stream(q.device)))
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
    T, C = x.shape
    _contig(x, "x")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    N = cu_seqlens.shape[0] - 1
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    cstride = _row_view(conv_pool, (3, C), "conv_pool")
    out = torch.empty((T, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    need = prefill_workspace_bytes(N, T, Hqk, Hv, dk, dv, mode)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = load_library().kda_prefill_conv if kda else load_library().gdn_prefill_conv
    _check(fn(N, T, Hqk, Hv, dk, dv, _ptr(x), _dtype(x), _ptr(_contig(conv_w, "conv_w")),
              _ptr(conv_b), _ptr(conv_pool), cstride, _dtype(conv_pool),
              _ptr(_contig(g, "g")), _ptr(_contig(beta, "beta")),
              _ptr(_contig(cu_seqlens, "cu_seqlens")), _ptr(_contig(slot_in, "slot_in")),
              _ptr(_contig(slot_out, "slot_out")), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _ptr(_contig(out, "out")), eps, scale, mode, _ptr(workspace),
              ws_bytes, _stream(x.device)))
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


def _ring_struct(ring):
    for k in ("d", "k", "rawv", "rawk", "g", "beta"):
        _contig(ring[k], f"ring[{k!r}]")
    return LaRing(ring["d"].shape[2], ring["d"].data_ptr(), ring["k"].data_ptr(),
                  ring["rawv"].data_ptr(), ring["rawk"].data_ptr(), ring["g"].data_ptr(),
                  ring["beta"].data_ptr())


def _verify(kda, x, g, beta, slots, n_tok, ssm_pool, ring, ring_base, *, Hqk, conv_w=None,
            conv_b=None, conv_pool=None, out=None, windows=None, eps=1e-6, scale=1.0):
    B, D, C = x.shape
    _contig(x, "x")
    rows, Hv, dv, dk = ssm_pool.shape
    if C != 2 * Hqk * dk + Hv * dv:
        raise ValueError(f"x has {C} channels, expected 2*Hqk*dk + Hv*dv")
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    cstride, cdt = 0, LA_F32
    if conv_w is not None:
        cstride = _row_view(conv_pool, (3, C), "conv_pool")
        cdt = _dtype(conv_pool)
        if windows is None:
            windows = torch.empty((B, D, 3, C), dtype=conv_pool.dtype, device=x.device)
    out = torch.empty((B, D, Hv, dv), dtype=x.dtype, device=x.device) if out is None else out
    r = _ring_struct(ring)
    fn = load_library().kda_verify if kda else load_library().gdn_verify
    _check(fn(B, D, _ptr(_contig(n_tok, "n_tok")), Hqk, Hv, dk, dv, _ptr(x), _dtype(x),
              _ptr(conv_w), _ptr(conv_b), _ptr(conv_pool), cstride, cdt, _ptr(_contig(g, "g")),
              _ptr(_contig(beta, "beta")), _ptr(_contig(slots, "slots")), rows, _ptr(ssm_pool),
              sstride, _dtype(ssm_pool), _ptr(_contig(out, "out")), _ptr(windows),
              ctypes.byref(r), _ptr(_contig(ring_base, "ring_base")), eps, scale,
              _stream(x.device)))
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
    rows, Hv, dv, dk = ssm_pool.shape
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    r = _ring_struct(ring)
    fn = load_library().kda_commit if kda else load_library().gdn_commit
    _check(fn(slots.shape[0], _ptr(_contig(accepted, "accepted")), Hv, dk, dv,
              _ptr(_contig(slots, "slots")), rows, _ptr(ssm_pool), sstride, _dtype(ssm_pool),
              _dtype(ring["d"]), ctypes.byref(r), _ptr(_contig(ring_base, "ring_base")), eps,
              _stream(ssm_pool.device)))


def kda_commit(accepted, slots, ssm_pool, ring, ring_base, eps=1e-6):
    """Exact commit: replays the first accepted[b] ring steps of each request
    from its pool row, in place."""
    _commit(True, accepted, slots, ssm_pool, ring, ring_base, eps)


def gdn_commit(accepted, slots, ssm_pool, ring, ring_base, eps=1e-6):
    """GDN exact commit; as :func:`kda_commit`."""
    _commit(False, accepted, slots, ssm_pool, ring, ring_base, eps)


def conv_window_scatter(windows, slots, step, conv_pool, mask=None):
    """conv_pool[slots[b]] = windows[b, step[b]] where mask[b] (uint8 or bool;
    None = all) and 0 <= step[b] < D."""
    B, D, three, C = windows.shape
    stride = _row_view(conv_pool, (3, C), "conv_pool")
    if mask is not None:
        mask = _contig(mask.to(torch.uint8), "mask")
    _check(load_library().conv_window_scatter(
        B, D, C, _ptr(mask), _ptr(_contig(slots, "slots")), _ptr(_contig(step, "step")),
        _ptr(_contig(windows, "windows")), _ptr(conv_pool), stride, _dtype(conv_pool),
        conv_pool.shape[0], _stream(conv_pool.device)))


def state_track_copy(src, dst, conv_pool, ssm_pool, mask=None):
    """Rows dst[b] of both pools become copies of rows src[b] where mask[b]."""
    crow = conv_pool[0].numel()
    srow = ssm_pool[0].numel()
    if not conv_pool[0].is_contiguous() or not ssm_pool[0].is_contiguous():
        raise ValueError("pool rows must be contiguous")
    if mask is not None:
        mask = _contig(mask.to(torch.uint8), "mask")
    _check(load_library().state_track_copy(
        src.shape[0], _ptr(mask), _ptr(_contig(src, "src")), _ptr(_contig(dst, "dst")),
        _ptr(conv_pool), conv_pool.stride(0), crow, _dtype(conv_pool), _ptr(ssm_pool),
        ssm_pool.stride(0), srow, _dtype(ssm_pool), ssm_pool.shape[0],
        _stream(ssm_pool.device)))


def _fold(kda, m, slots, ssm_pool, ring, ring_base, dst=None, q=None, out=None, eps=1e-6,
          scale=1.0):
    rows, Hv, dv, dk = ssm_pool.shape
    sstride = _row_view(ssm_pool, (Hv, dv, dk), "ssm_pool")
    B = slots.shape[0]
    if q is not None and out is None:
        out = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    r = _ring_struct(ring)
    fn = load_library().kda_ring_fold if kda else load_library().gdn_ring_fold
    _check(fn(B, _ptr(_contig(m, "m")), Hv, dk, dv, _ptr(_contig(slots, "slots")),
              _ptr(dst if dst is None else _contig(dst, "dst")), rows, _ptr(ssm_pool), sstride,
              _dtype(ssm_pool), _dtype(ring["d"]), ctypes.byref(r),
              _ptr(_contig(ring_base, "ring_base")), _ptr(q if q is None else _contig(q, "q")),
              _ptr(out), eps, scale, _stream(ssm_pool.device)))
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
