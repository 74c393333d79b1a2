"""fp64 CPU oracle for PaTH attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It is the plain definition of the
method (see ``path_oracle.c`` for the passages it follows), compiled with gcc
and called through ctypes.  It imports nothing from the HIP library and the HIP
library imports nothing from it.

Parity of every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, textbook routines and brute force; see that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "path_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpath_oracle.so")

_lib = None


def build(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no contraction)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str = LIB_PATH):
    """Load (building first if absent) the oracle library."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_path_logits.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, dp]
    lib.oracle_path_logits.restype = None
    lib.oracle_path_walk.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, dp]
    lib.oracle_path_walk.restype = None
    lib.oracle_path_attn_rows.argtypes = [
        dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, dp, dp,
        ctypes.c_int]
    lib.oracle_path_attn_rows.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def path_logits(q, k, w, beta, logf=None, scale=1.0, lib=None):
    """Logit matrix of one head, [T, T]; -inf above the diagonal.

    q, k, w: [T, d]; beta, logf: [T].  With scale=1 and logf=None the entries
    are the raw path logits c_ij = k_j^T H_{j+1}...H_i q_i.
    """
    lib = lib or load()
    q, k, w, beta = _f64(q), _f64(k), _f64(w), _f64(beta)
    logf = None if logf is None else _f64(logf)
    T, d = q.shape
    S = np.empty((T, T), dtype=np.float64)
    lib.oracle_path_logits(_ptr(q), _ptr(k), _ptr(w), _ptr(beta), _ptr(logf),
                           T, d, float(scale), _ptr(S))
    return S


def path_walk(q, w, beta, i, lib=None):
    """Walked query vectors of row i: result[m] = H_{i-m+1}...H_i q_i, m=0..i."""
    lib = lib or load()
    q, w, beta = _f64(q), _f64(w), _f64(beta)
    T, d = q.shape
    Z = np.empty((i + 1, d), dtype=np.float64)
    lib.oracle_path_walk(_ptr(q), _ptr(w), _ptr(beta), int(i), d, _ptr(Z))
    return Z


def path_attn_rows(q, k, v, w, beta, logf, scale, rows, n_threads=0, lib=None):
    """Outputs and lse for selected rows.

    q, k, v, w: [n_heads, T, d]; beta, logf: [n_heads, T] (logf may be None);
    rows: int array [R, 2] of (head, query index).  Returns (out [R, d],
    lse [R]) in fp64.
    """
    lib = lib or load()
    q, k, v, w, beta = _f64(q), _f64(k), _f64(v), _f64(w), _f64(beta)
    logf = None if logf is None else _f64(logf)
    n_heads, T, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
    R = rows.shape[0]
    out = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    rc = lib.oracle_path_attn_rows(
        _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(beta), _ptr(logf), n_heads,
        T, d, float(scale), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        R, _ptr(out), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError("oracle: row index out of range")
    return out, lse


def path_attn(q, k, v, w, beta, logf=None, scale=None, n_threads=0, lib=None):
    """Full forward pass: q, k, v, w [..., T, d] and beta/logf [..., T].

    Returns (out [..., T, d], lse [..., T]) in fp64.  scale defaults to
    1/sqrt(d).
    """
    q = np.asarray(q)
    lead = q.shape[:-2]
    T, d = q.shape[-2:]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_heads = int(np.prod(lead)) if lead else 1
    r = lambda x: None if x is None else np.asarray(x).reshape(n_heads, T, -1)
    rb = lambda x: None if x is None else np.asarray(x).reshape(n_heads, T)
    rows = np.stack(np.meshgrid(np.arange(n_heads), np.arange(T),
                                indexing="ij"), -1).reshape(-1, 2)
    out, lse = path_attn_rows(r(q), r(k), r(v), r(w), rb(beta), rb(logf),
                              scale, rows, n_threads=n_threads, lib=lib)
    return out.reshape(*lead, T, d), lse.reshape(*lead, T)


def max_threads(lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_max_threads())
