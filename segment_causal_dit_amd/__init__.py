"""MI355X (gfx950) segment-wise causal joint attention over a persistent KV cache.

The compute lives in libsegcausal.so (hand-written HIP, C ABI in
include/segcausal.h); this package is its thin Python binding. The binding is
loaded on first use of any of its names and raises ImportError if the library
has not been built (`python -m segment_causal_dit_amd.build`); there is no
fallback implementation.
"""

_NAMES = (
    "SEGC_OK", "SEGC_EINVAL", "SEGC_EUNSUPPORTED", "SEGC_EHIP", "SEGC_BF16", "SEGC_INT8",
    "KVCache", "SegcError", "abi_version", "camera_cross_attn", "kv_archive_fetch", "kv_archive_store", "kv_cache_append",
    "kv_window_dequant", "rope3d_apply",
    "segcausal_joint_attn", "segcausal_joint_attn_bwd", "segcausal_joint_attn_bwd_noalloc",
    "attn_workspace_bytes", "w8a16_linear", "window_select", "LIB_PATH", "EXPORTS", "ABI_VERSION",
)


def __getattr__(name):
    if name in _NAMES:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)


__all__ = list(_NAMES)
