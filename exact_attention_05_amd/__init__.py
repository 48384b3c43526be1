"""MI355X-native exact attention: FA-2 style forward, split-K decode (over a
dense or a paged cache), recomputation backward and an FP8 (E4M3) forward, as hand-written HIP kernels for gfx950 behind a
C ABI (``libattn.so``, declared in ``include/attn.h``).

The Python names mirror the C entry points; the shared library is loaded on
first use, and every call fails loudly when it is missing.
"""

__all__ = [
    "attn_fwd",
    "attn_fwd_merge",
    "attn_fwd_splitk_decode",
    "attn_fwd_splitk_decode_paged",
    "attn_fwd_splitk_decode_noalloc",
    "attn_bwd",
    "attn_bwd_atomic_dq",
    "attn_quantize_fp8",
    "attn_fwd_fp8",
    "attn_merge",
    "attn_decode_workspace_bytes",
    "attn_bwd_workspace_bytes",
    "attn_bwd_atomic_workspace_bytes",
    "attn_status_string",
    "AttnError",
    "library_path",
    "split_decode_workspace",
    "raw_library",
]


def __getattr__(name):
    if name in __all__:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
