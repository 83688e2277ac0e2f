"""MI355X-native fused attention forward and latent-cache MLA decode.

The compute lives in ``libmla_attn.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/mla_attn.h``).  ``binding`` is a thin ctypes layer with
the same function names that only marshals torch tensors into device
pointers and the current HIP stream.  Importing this package does not load
the library; the first call into ``binding`` does, and raises if it is
missing.  There is no CPU fallback.
"""

__all__ = [
    "attn_fwd",
    "attn_fwd_chunk",
    "mla_decode_fwd",
    "mla_decode_workspace_size",
    "mla_decode_fwd_noalloc",
    "mla_decode_v_workspace_size",
    "mla_decode_fwd_v",
    "mla_combine",
    "mla_absorb_q",
    "mla_up_proj_v",
    "mla_status_string",
    "MlaError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
