"""PaTH attention for AMD Instinct MI355X (gfx950): forward, backward, decoding
and the w / beta producer.

The computation lives in the HIP library ``libpath_attn.so`` (C ABI declared
in ``include/path_attn.h``).  This package is a thin ctypes binding: it checks
and marshals torch tensors (device pointers, the current HIP stream) and
raises on a non-zero status.  There is no CPU fallback: if the library is
missing or no GPU is present the calls raise.
"""
from .binding import (  # noqa: F401
    BF16,
    DecodeCache,
    F32,
    NOALLOC_MAX_BYTES,
    NO_SKIP,
    PRECISE,
    PathAttnError,
    chunk_prep,
    library_path,
    load_library,
    path_attn_bwd,
    path_attn_bwd_varlen,
    path_attn_bwd_varlen_workspace_bytes,
    path_attn_bwd_workspace_bytes,
    path_attn_bwd_workspace_bytes_window,
    path_attn_chunk_prep,
    path_attn_decode_step,
    path_attn_fwd,
    path_attn_fwd_noalloc,
    path_attn_fwd_partial,
    path_attn_fwd_varlen,
    path_attn_prefill_cache,
    path_attn_prepare,
    path_attn_stream,
    path_attn_varlen_workspace_bytes,
    path_attn_wbeta,
    path_attn_workspace_bytes,
    strerror,
    version,
)

__all__ = [
    "BF16", "DecodeCache", "F32", "NOALLOC_MAX_BYTES", "NO_SKIP", "PRECISE", "PathAttnError", "chunk_prep", "library_path",
    "load_library", "path_attn_bwd", "path_attn_bwd_varlen",
    "path_attn_bwd_varlen_workspace_bytes", "path_attn_bwd_workspace_bytes",
    "path_attn_bwd_workspace_bytes_window",
    "path_attn_chunk_prep", "path_attn_decode_step", "path_attn_fwd", "path_attn_fwd_noalloc", "path_attn_fwd_partial",
    "path_attn_fwd_varlen",
    "path_attn_prefill_cache", "path_attn_prepare", "path_attn_stream",
    "path_attn_varlen_workspace_bytes", "path_attn_wbeta", "path_attn_workspace_bytes", "strerror",
    "version",
]
