"""MI355X-native linear-attention recurrent-state path.

Kimi Delta Attention (per-channel decay) and Gated DeltaNet (per-head scalar
gate) decode steps, the kernel-size-4 depthwise causal short conv, and the
chunked prefill, all keyed by slot indices into slot-indexed state pools.
The compute lives in hand-written HIP kernels for gfx950 behind the C ABI in
``include/la.h`` (``libla.so``); :mod:`.binding` marshals torch tensors and
streams into that ABI.  Importing a kernel entry point loads ``libla.so`` and
raises if it has not been built -- there is no CPU fallback.
"""
from __future__ import annotations

_BINDING_NAMES = {
    "kda_decode_step", "gdn_decode_step", "shortconv_update", "shortconv_prefill",
    "kda_prefill_chunked", "kda_prefill_chunked_noalloc", "gdn_prefill_chunked", "kda_prefill_conv", "gdn_prefill_conv",
    "prefill_workspace_bytes", "kda_prefill_workspace_bytes", "gdn_prefill_workspace_bytes",
    "pool_bytes", "ring_bytes", "version", "LAError", "load_library", "library_path",
    "kda_verify", "gdn_verify", "kda_commit", "gdn_commit", "conv_window_scatter",
    "state_track_copy", "new_ring", "kda_ring_fold", "gdn_ring_fold",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
