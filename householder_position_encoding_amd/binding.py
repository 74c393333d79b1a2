"""ctypes binding of libpath_attn (argument marshalling only).

Every entry point of ``include/path_attn.h`` has a function of the same name
here taking raw integers (device addresses) exactly like the C ABI, plus the
torch-level conveniences ``path_attn_fwd`` accepts (tensors in, tensors out).
All arithmetic happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_PKG, "libpath_attn.so")

F32 = 0
BF16 = 1

STATUS = {0: "PATH_ATTN_OK", 1: "PATH_ATTN_EINVAL", 2: "PATH_ATTN_EUNSUPPORTED",
          3: "PATH_ATTN_EHIP"}

_lib = None


class PathAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status)})")


def library_path() -> str:
    return os.environ.get("PATH_ATTN_LIB", _LIB_FILE)


def load_library():
    """Load libpath_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"libpath_attn.so not found at {path}; build it with "
            "`python -m householder_position_encoding_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, ci, fp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
    lib.path_attn_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.path_attn_workspace_bytes.restype = sz
    lib.path_attn_fwd.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, ci, ci, ci, ci,
                                  ci, vp, sz, vp]
    lib.path_attn_fwd.restype = ci
    lib.path_attn_fwd_ex.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, ci, ci, ci, ci,
                                     ci, ctypes.c_float, ctypes.c_uint, vp, sz, vp]
    lib.path_attn_fwd_ex.restype = ci
    lib.path_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, ci, ci, ci, ci, ci,
                                          ctypes.c_float, ctypes.c_uint, vp]
    lib.path_attn_fwd_noalloc.restype = ci
    lib.path_attn_fwd_partial.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, ci, ci, ci, ci, ci, ci,
                                          ctypes.c_float, ctypes.c_uint, vp, sz, vp]
    lib.path_attn_fwd_partial.restype = ci
    lib.path_attn_chunk_prep.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, fp, fp,
                                         fp, ci, ci, ci, ci, ci, vp, sz, vp]
    lib.path_attn_chunk_prep.restype = ci
    lib.path_attn_prepare.argtypes = [vp, vp, vp, vp, fp, fp, ci, ci, ci, ci, ci,
                                      vp, sz, vp]
    lib.path_attn_prepare.restype = ci
    lib.path_attn_stream.argtypes = [vp, sz, ci, vp, fp, ci, ci, ci, ci, ci, vp]
    lib.path_attn_stream.restype = ci
    lib.path_attn_stream_ex.argtypes = [vp, sz, ci, ctypes.c_float, ctypes.c_uint, vp, vp,
                                        fp, ci, ci, ci, ci, ci, vp]
    lib.path_attn_stream_ex.restype = ci
    lib.path_attn_prefill_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.path_attn_prefill_workspace_bytes.restype = sz
    lib.path_attn_prefill_cache.argtypes = [vp, vp, vp, fp, fp, vp, vp, vp, ci, ci, ci, ci,
                                            ci, ci, ci, vp, sz, vp]
    lib.path_attn_prefill_cache.restype = ci
    lib.path_attn_decode_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.path_attn_decode_workspace_bytes.restype = sz
    lib.path_attn_decode_step.argtypes = [vp, vp, vp, vp, fp, fp, vp, vp, vp, ci, vp, fp,
                                          ci, ci, ci, ci, ci, ci, ctypes.c_float, vp, sz, vp]
    lib.path_attn_decode_step.restype = ci
    lib.path_attn_wbeta.argtypes = [vp, vp, vp, fp, vp, fp, vp, fp, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.path_attn_wbeta.restype = ci
    lib.path_attn_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.path_attn_bwd_workspace_bytes.restype = sz
    lib.path_attn_bwd_workspace_bytes_window.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.path_attn_bwd_workspace_bytes_window.restype = sz
    lib.path_attn_bwd.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, vp, vp, vp, fp,
                                  fp, ci, ci, ci, ci, ci, ctypes.c_float, vp, sz, vp]
    lib.path_attn_bwd.restype = ci
    lib.path_attn_bwd_ex.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, vp, vp, vp, fp,
                                     fp, ci, ci, ci, ci, ci, ctypes.c_float, ctypes.c_uint, vp, sz,
                                     vp]
    lib.path_attn_bwd_ex.restype = ci
    lib.path_attn_varlen_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.path_attn_varlen_workspace_bytes.restype = sz
    lib.path_attn_fwd_varlen.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, vp, ci, ci, ci,
                                         ci, ci, ctypes.c_float, ctypes.c_uint, vp, sz, vp]
    lib.path_attn_fwd_varlen.restype = ci
    lib.path_attn_bwd_varlen_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.path_attn_bwd_varlen_workspace_bytes.restype = sz
    lib.path_attn_bwd_varlen.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, vp, vp,
                                         vp, fp, fp, vp, vp, ci, ci, ci, ci, ci,
                                         ctypes.c_float, vp, sz, vp]
    lib.path_attn_bwd_varlen.restype = ci
    lib.path_attn_strerror.argtypes = [ci]
    lib.path_attn_strerror.restype = ctypes.c_char_p
    lib.path_attn_version.argtypes = []
    lib.path_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().path_attn_strerror(int(status)).decode()


def version() -> str:
    return load_library().path_attn_version().decode()


def path_attn_workspace_bytes(B: int, H: int, T: int, d: int, dtype: int) -> int:
    return int(load_library().path_attn_workspace_bytes(B, H, T, d, dtype))


# ---------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v/w must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _common(q, k, v, w, beta, logf):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (no CPU path)")
    for name, t in (("k", k), ("v", v), ("w", w)):
        _check(t, name, q.shape, q.dtype, dev)
    _check(q, "q", q.shape, q.dtype, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    if logf is not None:
        _check(logf, "logf", (B, H, T), torch.float32, dev)
    return B, H, T, d, _dtype_code(q)


def path_attn_fwd(q, k, v, w, beta, logf=None, out=None, lse=None,
                  workspace=None, stream=None, scale=None, flags=0):
    """PaTH attention forward on the GPU.

    q, k, v, w: [B, H, T, d] bf16 or fp32 CUDA tensors (same dtype);
    beta: [B, H, T] fp32; logf: optional [B, H, T] fp32 (PaTH-FoX).
    Returns (out [B, H, T, d] in q's dtype, lse [B, H, T] fp32).  A workspace
    (uint8 CUDA tensor of at least path_attn_workspace_bytes bytes) may be
    passed to avoid an allocation.  scale: softmax scale (None: 1/sqrt(d));
    flags: 0, or NO_SKIP and/or PRECISE (path_attn_fwd_ex).
    """
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", (B, H, T), torch.float32, q.device)
    need = lib.path_attn_workspace_bytes(B, H, T, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.path_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
                              _ptr(logf), _ptr(out), _ptr(lse), B, H, T, d, dt,
                              0.0 if scale is None else float(scale), int(flags),
                              _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_fwd_ex")
    return out, lse


def path_attn_fwd_partial(q, k, v, w, beta, logf=None, d_path=None, out=None, lse=None,
                          workspace=None, stream=None, scale=None, flags=0):
    """Partial PaTH (path_attn_fwd_partial): the factors act on the leading
    d_path coordinates only (w is not read beyond them); d_path is d or d // 2
    (None: d // 2).  Other arguments as path_attn_fwd."""
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    lib = load_library()
    d_path = d // 2 if d_path is None else int(d_path)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", (B, H, T), torch.float32, q.device)
    need = lib.path_attn_workspace_bytes(B, H, T, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.path_attn_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
                                   _ptr(out), _ptr(lse), B, H, T, d, d_path, dt,
                                   0.0 if scale is None else float(scale), int(flags),
                                   _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_fwd_partial")
    return out, lse


NOALLOC_MAX_BYTES = 64 << 20   # PATH_ATTN_NOALLOC_MAX_BYTES of the header


def path_attn_fwd_noalloc(q, k, v, w, beta, logf=None, out=None, lse=None, stream=None,
                          scale=None, flags=0):
    """path_attn_fwd_noalloc: the forward with the library's fixed device
    array as its workspace (no workspace argument, nothing allocated by the
    call; problems up to NOALLOC_MAX_BYTES of workspace).  out and lse are
    allocated here when not given; pass them to allocate nothing.  Calls on
    one GPU share the array and must not overlap."""
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", (B, H, T), torch.float32, q.device)
    st = lib.path_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
                                   _ptr(out), _ptr(lse), B, H, T, d, dt,
                                   0.0 if scale is None else float(scale), int(flags),
                                   _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_fwd_noalloc")
    return out, lse


def path_attn_prepare(q, k, v, w, beta, logf=None, workspace=None, stream=None):
    """First phase of path_attn_fwd: fill `workspace` (allocated if None) with
    the gate prefix and the chunk preparation.  Returns the workspace."""
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    lib = load_library()
    need = lib.path_attn_workspace_bytes(B, H, T, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.path_attn_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
                               _ptr(logf), B, H, T, d, dt, _ptr(workspace),
                               workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_prepare")
    return workspace


NO_SKIP = 1   # PATH_ATTN_NO_SKIP
PRECISE = 2   # PATH_ATTN_PRECISE


def path_attn_stream(workspace, use_gate, out, lse, stream=None, flags=0,
                     skipped=None, scale=None):
    """Second phase of path_attn_fwd: the streaming scan over a workspace
    filled by path_attn_prepare for the same shapes; writes out and lse.

    flags=NO_SKIP computes every key block (no exact forget-gate skip);
    skipped, an int64 device tensor of one element, receives += the number of
    skipped (wave, key block) steps (path_attn_stream_ex)."""
    torch = _torch()
    B, H, T, d = out.shape
    dt = _dtype_code(out)
    _check(lse, "lse", (B, H, T), torch.float32, out.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if skipped is not None:
        _check(skipped, "skipped", (1,), torch.int64, out.device)
    lib = load_library()
    st = lib.path_attn_stream_ex(_ptr(workspace), workspace.numel(), int(bool(use_gate)),
                                 0.0 if scale is None else float(scale), int(flags),
                                 _ptr(skipped), _ptr(out), _ptr(lse),
                                 B, H, T, d, dt, _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_stream_ex")
    return out, lse


def chunk_prep(q, k, v, w, beta, logf=None, stream=None):
    """Run only the chunk preparation and return its unpacked fp32 results:
    dict(qa [B,H,T,d], kb [B,H,T,d], m [B,H,N,d,d], al [B,H,N,64,64],
    lam [B,H,T] or None)."""
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    lib = load_library()
    N = T // 64
    f = dict(dtype=torch.float32, device=q.device)
    qa = torch.empty((B, H, T, d), **f)
    kb = torch.empty((B, H, T, d), **f)
    m = torch.empty((B, H, N, d, d), **f)
    al = torch.empty((B, H, N, 64, 64), **f)
    lam = torch.empty((B, H, T), **f) if logf is not None else None
    need = lib.path_attn_workspace_bytes(B, H, T, d, dt)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.path_attn_chunk_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta),
                                  _ptr(logf), _ptr(qa), _ptr(kb), _ptr(m), _ptr(al),
                                  _ptr(lam), B, H, T, d, dt, _ptr(ws), ws.numel(),
                                  _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_chunk_prep")
    return dict(qa=qa, kb=kb, m=m, al=al, lam=lam)


def path_attn_chunk_prep(*args):
    """Raw C-ABI call with integer pointers (see include/path_attn.h)."""
    return int(load_library().path_attn_chunk_prep(*args))


# ---------------------------------------------------------------- decoding

class DecodeCache:
    """Caller-side caches for decoding with in-place key refinement.

    kcache [B, H, T_cap, d] (kc_dtype), vcache [B, H, T_cap, d] (dtype),
    gcache [B, H, T_cap] float64 (only with the forget gate), plus the
    decode workspace.  `length` is the number of positions filled.
    """

    def __init__(self, B, H, T_cap, d, dtype, kc_dtype=None, fox=False, device="cuda"):
        torch = _torch()
        self.B, self.H, self.T_cap, self.d = B, H, T_cap, d
        self.dtype = dtype
        self.kc_dtype = torch.float32 if kc_dtype is None else kc_dtype
        self.fox = fox
        self.kcache = torch.zeros((B, H, T_cap, d), dtype=self.kc_dtype, device=device)
        self.vcache = torch.zeros((B, H, T_cap, d), dtype=dtype, device=device)
        self.gcache = torch.zeros((B, H, T_cap), dtype=torch.float64, device=device) if fox else None
        need = load_library().path_attn_decode_workspace_bytes(B, H, T_cap, d)
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        self.length = 0


def _code_of(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dtype}")


def path_attn_prefill_cache(cache, k, v, w, beta, logf=None, workspace=None, stream=None):
    """Fill positions 0..L-1 of `cache` from a prompt (k, v, w [B, H, L, d];
    beta, logf [B, H, L]); L must be a multiple of 64."""
    torch = _torch()
    B, H, L, d = k.shape
    dev = k.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (no CPU path)")
    for name, t in (("k", k), ("v", v), ("w", w)):
        _check(t, name, (cache.B, cache.H, L, cache.d), cache.dtype, dev)
    _check(beta, "beta", (B, H, L), torch.float32, dev)
    if (logf is not None) != cache.fox:
        raise ValueError("logf must be given exactly when the cache has a gate")
    if logf is not None:
        _check(logf, "logf", (B, H, L), torch.float32, dev)
    lib = load_library()
    need = lib.path_attn_prefill_workspace_bytes(B, H, L, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.path_attn_prefill_cache(
        _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(cache.kcache),
        _ptr(cache.vcache), _ptr(cache.gcache), B, H, L, cache.T_cap, d,
        _code_of(cache.dtype), _code_of(cache.kc_dtype), _ptr(workspace), workspace.numel(),
        _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_prefill_cache")
    cache.length = L
    return cache


def path_attn_decode_step(cache, q, k, v, w, beta, logf=None, out=None, lse=None, stream=None,
                          scale=None):
    """One decode step at position cache.length: q, k, v, w [B, H, d];
    beta, logf [B, H].  Returns (out [B, H, d], lse [B, H])."""
    torch = _torch()
    B, H, d = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU (no CPU path)")
    for name, t in (("q", q), ("k", k), ("v", v), ("w", w)):
        _check(t, name, (cache.B, cache.H, cache.d), cache.dtype, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    if (logf is not None) != cache.fox:
        raise ValueError("logf must be given exactly when the cache has a gate")
    if logf is not None:
        _check(logf, "logf", (B, H), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    lib = load_library()
    st = lib.path_attn_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), _ptr(cache.kcache),
        _ptr(cache.vcache), _ptr(cache.gcache), cache.length, _ptr(out), _ptr(lse), B, H,
        cache.T_cap, d, _code_of(cache.dtype), _code_of(cache.kc_dtype),
        0.0 if scale is None else float(scale),
        _ptr(cache.workspace), cache.workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_decode_step")
    cache.length += 1
    return out, lse


# ---------------------------------------------------------------- backward

def path_attn_wbeta(x, wd, wu, cw, u, ub, H: int, d: int, w=None, beta=None, stream=None):
    """The w / beta producer (path_attn_wbeta): x [B, T, Dm] bf16 hidden
    states, wd [R, Dm], wu [H*d, R], u [H, Dm] bf16, cw [H*d, 3] and ub [H]
    float32 -> (w [B, H, T, d] bf16, beta [B, H, T] float32)."""
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be [B, T, Dm]")
    B, T, Dm = x.shape
    R = wd.shape[0]
    _check(x, "x", (B, T, Dm), torch.bfloat16, x.device)
    _check(wd, "wd", (R, Dm), torch.bfloat16, x.device)
    _check(wu, "wu", (H * d, R), torch.bfloat16, x.device)
    _check(cw, "cw", (H * d, 3), torch.float32, x.device)
    _check(u, "u", (H, Dm), torch.bfloat16, x.device)
    _check(ub, "ub", (H,), torch.float32, x.device)
    if w is None:
        w = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=x.device)
    if beta is None:
        beta = torch.empty((B, H, T), dtype=torch.float32, device=x.device)
    _check(w, "w", (B, H, T, d), torch.bfloat16, x.device)
    _check(beta, "beta", (B, H, T), torch.float32, x.device)
    lib = load_library()
    st = lib.path_attn_wbeta(_ptr(x), _ptr(wd), _ptr(wu), _ptr(cw), _ptr(u), _ptr(ub), _ptr(w),
                             _ptr(beta), B, T, Dm, R, H, d, 1, _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_wbeta")
    return w, beta


def path_attn_bwd_workspace_bytes(B: int, H: int, T: int, d: int, dtype: int) -> int:
    return int(load_library().path_attn_bwd_workspace_bytes(B, H, T, d, dtype))


def path_attn_bwd_workspace_bytes_window(B: int, H: int, T: int, d: int, dtype: int,
                                         window: int) -> int:
    return int(load_library().path_attn_bwd_workspace_bytes_window(B, H, T, d, dtype, window))


def path_attn_bwd(q, k, v, w, beta, logf, out, lse, dout, dlse=None, scale=None,
                  workspace=None, stream=None, window=None, flags=0):
    """Gradients of <dout, out> + <dlse, lse> for the forward of path_attn_fwd
    (out, lse: that forward's outputs).  Returns (dq, dk, dv, dw, dbeta,
    dlogf); dlogf is None without the gate.  Any T >= 1 (padded inside the
    library as in the forward).  Without a workspace, one of the smallest
    size is allocated, or with window given the size of
    path_attn_bwd_workspace_bytes_window (0: the whole sweep as one window,
    the fastest); a larger workspace selects longer windows.  flags: 0 or
    NO_SKIP (path_attn_bwd_ex: every block computed, no forget-gate skip)."""
    torch = _torch()
    B, H, T, d, dt = _common(q, k, v, w, beta, logf)
    _check(out, "out", q.shape, q.dtype, q.device)
    _check(dout, "dout", q.shape, q.dtype, q.device)
    _check(lse, "lse", (B, H, T), torch.float32, q.device)
    if dlse is not None:
        _check(dlse, "dlse", (B, H, T), torch.float32, q.device)
    lib = load_library()
    dq, dk, dv, dw = (torch.empty_like(q) for _ in range(4))
    dbeta = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    dlogf = None if logf is None else torch.empty_like(dbeta)
    if window is None:
        need = lib.path_attn_bwd_workspace_bytes(B, H, T, d, dt)
    else:
        need = lib.path_attn_bwd_workspace_bytes_window(B, H, T, d, dt, int(window))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.path_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
                              _ptr(out), _ptr(lse), _ptr(dout), _ptr(dlse), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(dw), _ptr(dbeta), _ptr(dlogf), B, H, T, d, dt,
                              0.0 if scale is None else float(scale), int(flags),
                              _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_bwd_ex")
    return dq, dk, dv, dw, dbeta, dlogf


# ------------------------------------------------- strided and packed batches

def path_attn_varlen_workspace_bytes(B: int, H: int, T: int, d: int, dtype: int) -> int:
    return int(load_library().path_attn_varlen_workspace_bytes(B, H, T, d, dtype))


def path_attn_bwd_varlen_workspace_bytes(B: int, H: int, T: int, d: int, dtype: int) -> int:
    return int(load_library().path_attn_bwd_varlen_workspace_bytes(B, H, T, d, dtype))


class _Views:
    """Shapes and (s_b, s_h, s_t) element strides of the tensors of a varlen
    call.  Without cu_seqlens the vectors are [B, H, T, d] views and the
    scalars [B, H, T] views; with cu_seqlens (int32 CUDA tensor [B + 1]) the
    vectors are token-major [total, H, d] views and the scalars [total, H]."""

    def __init__(self, q, cu_seqlens, max_seqlen):
        torch = _torch()
        if q.device.type != "cuda":
            raise ValueError("tensors must live on a GPU (no CPU path)")
        self.device, self.dtype = q.device, q.dtype
        self.packed = cu_seqlens is not None
        if self.packed:
            if q.dim() != 3:
                raise ValueError("with cu_seqlens, q must be [total, H, d]")
            if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or \
                    cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
                raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor on q's device")
            self.B = cu_seqlens.numel() - 1
            if self.B < 1:
                raise ValueError("cu_seqlens needs at least two entries")
            total, self.H, self.d = q.shape
            if max_seqlen is None:   # host read of the lengths (synchronises)
                max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
            self.T = int(max_seqlen)
            self.vshape, self.sshape = tuple(q.shape), (total, self.H)
        else:
            if q.dim() != 4:
                raise ValueError("q must be [B, H, T, d]")
            self.B, self.H, self.T, self.d = q.shape
            self.vshape, self.sshape = tuple(q.shape), (self.B, self.H, self.T)

    def strides(self, t, name, vector, dtype=None):
        torch = _torch()
        if t is None:
            return (0, 0, 0)
        want = dtype if dtype is not None else (self.dtype if vector else torch.float32)
        shape = self.vshape if vector else self.sshape
        if t.device != self.device:
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        if t.dtype != want:
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
        st = t.stride()
        if vector and st[-1] != 1 and t.shape[-1] > 1:
            raise ValueError(f"{name}: the d elements of a row must be contiguous")
        if self.packed:
            return (0, st[1], st[0])
        return (st[0], st[1], st[2])

    def new_vector(self):
        return _torch().zeros(self.vshape, dtype=self.dtype, device=self.device)

    def new_scalar(self):
        return _torch().zeros(self.sshape, dtype=_torch().float32, device=self.device)


def _stride_array(triples):
    flat = [int(x) for tr in triples for x in tr]
    return (ctypes.c_longlong * len(flat))(*flat)


def path_attn_fwd_varlen(q, k, v, w, beta, logf=None, cu_seqlens=None, max_seqlen=None,
                         out=None, lse=None, scale=None, flags=0, workspace=None, stream=None):
    """PaTH attention forward on strided views or packed sequences
    (path_attn_fwd_varlen of the C ABI).

    Without cu_seqlens: q, k, v, w are [B, H, T, d] views with any strides
    (each row's d elements contiguous), beta and logf [B, H, T] views.  With
    cu_seqlens (int32 CUDA [B + 1], the start of each sequence in tokens):
    q, k, v, w are token-major [total, H, d] views, beta and logf [total, H],
    and each sequence is attended on its own; max_seqlen is the longest
    sequence (read from cu_seqlens, with a synchronisation, if None).
    Returns (out, lse) of the vector and scalar shapes (new zero-filled
    tensors unless given; rows outside every sequence are not written).
    """
    V = _Views(q, cu_seqlens, max_seqlen)
    out = V.new_vector() if out is None else out
    lse = V.new_scalar() if lse is None else lse
    tensors = [(q, "q", True), (k, "k", True), (v, "v", True), (w, "w", True),
               (out, "out", True), (beta, "beta", False), (logf, "logf", False),
               (lse, "lse", False)]
    strides = _stride_array(V.strides(t, n, vec) for t, n, vec in tensors)
    lib = load_library()
    dt = _dtype_code(q)
    need = lib.path_attn_varlen_workspace_bytes(V.B, V.H, V.T, V.d, dt)
    if workspace is None:
        workspace = _torch().empty(max(need, 256), dtype=_torch().uint8, device=q.device)
    st = lib.path_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
                                  _ptr(out), _ptr(lse), strides, _ptr(cu_seqlens), V.B, V.H,
                                  V.T, V.d, dt, 0.0 if scale is None else float(scale),
                                  int(flags), _ptr(workspace), workspace.numel(),
                                  _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_fwd_varlen")
    return out, lse


def path_attn_bwd_varlen(q, k, v, w, beta, logf, out, lse, dout, dlse=None, cu_seqlens=None,
                         max_seqlen=None, scale=None, workspace=None, stream=None):
    """Backward of path_attn_fwd_varlen (path_attn_bwd_varlen of the C ABI),
    with the same views and cu_seqlens.  Returns (dq, dk, dv, dw, dbeta,
    dlogf) as new zero-filled tensors of the vector and scalar shapes; dlogf
    is None without the gate."""
    V = _Views(q, cu_seqlens, max_seqlen)
    dq, dk, dv, dw = (V.new_vector() for _ in range(4))
    dbeta = V.new_scalar()
    dlogf = None if logf is None else V.new_scalar()
    tensors = [(q, "q", True), (k, "k", True), (v, "v", True), (w, "w", True),
               (out, "out", True), (dout, "dout", True), (dq, "dq", True), (dk, "dk", True),
               (dv, "dv", True), (dw, "dw", True), (beta, "beta", False),
               (logf, "logf", False), (lse, "lse", False), (dlse, "dlse", False),
               (dbeta, "dbeta", False), (dlogf, "dlogf", False)]
    strides = _stride_array(V.strides(t, n, vec) for t, n, vec in tensors)
    lib = load_library()
    dt = _dtype_code(q)
    need = lib.path_attn_bwd_varlen_workspace_bytes(V.B, V.H, V.T, V.d, dt)
    if workspace is None:
        workspace = _torch().empty(max(need, 256), dtype=_torch().uint8, device=q.device)
    st = lib.path_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf),
                                  _ptr(out), _ptr(lse), _ptr(dout), _ptr(dlse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _ptr(dw), _ptr(dbeta), _ptr(dlogf),
                                  strides, _ptr(cu_seqlens), V.B, V.H, V.T, V.d, dt,
                                  0.0 if scale is None else float(scale), _ptr(workspace),
                                  workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise PathAttnError(st, "path_attn_bwd_varlen")
    return dq, dk, dv, dw, dbeta, dlogf
