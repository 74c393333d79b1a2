"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments before any
HIP call (these calls never launch anything, so no GPU is needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import householder_position_encoding_amd as pa
from householder_position_encoding_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "path_attn.h")

OK, EINVAL, EUNSUP, EHIP = 0, 1, 2, 3
FAKE = 0x100000   # an aligned, non-null address; never dereferenced: every call
                  # below fails validation, which runs before any HIP call


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(path_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    syms = declared_symbols()
    assert {"path_attn_fwd", "path_attn_workspace_bytes", "path_attn_strerror",
            "path_attn_chunk_prep", "path_attn_version", "path_attn_prepare",
            "path_attn_stream"} <= set(syms)
    for s in syms:
        assert hasattr(lib, s), f"libpath_attn.so does not export {s}"


def test_version_and_strerror():
    assert "gfx950" in pa.version()
    for st in (OK, EINVAL, EUNSUP, EHIP):
        assert pa.strerror(st)
    assert pa.strerror(99) == "unknown status"


@pytest.mark.parametrize("dtype,esize", [(pa.F32, 4), (pa.BF16, 2)])
@pytest.mark.parametrize("B,H,T,d", [(1, 2, 256, 64), (2, 16, 16384, 64), (4, 8, 8192, 128)])
def test_workspace_bytes(dtype, esize, B, H, T, d):
    n = pa.path_attn_workspace_bytes(B, H, T, d, dtype)
    BH, N = B * H, T // 64
    # <-Q (fp32), the three per-chunk operands, 3 of 4 diagonal-logit tiles (fp32), gate,
    # two float32 skip bounds per chunk; bf16 also ->K's rounding remainders
    expect = (BH * T * d * 4 + BH * N * (2 * 64 * d + d * d) * esize + BH * N * 3 * 64 * 16 * 4
              + BH * T * 4 + BH * N * 2 * 4 + (BH * T * d * 2 if dtype == pa.BF16 else 0))
    assert expect <= n <= expect + 6 * 256


@pytest.mark.parametrize("args", [(0, 1, 64, 64, 1), (1, 0, 64, 64, 1), (1, 1, 0, 64, 1),
                                  (1, 1, 64, 96, 1), (1, 1, 64, 64, 7),
                                  (1, 1, 64, -64, 0), (1 << 16, 1 << 10, 1024, 64, 1)])
def test_workspace_bytes_rejects(args):
    assert pa.path_attn_workspace_bytes(*args) == 0


@pytest.mark.parametrize("dtype,esize", [(pa.F32, 4), (pa.BF16, 2)])
@pytest.mark.parametrize("T", [1, 63, 65, 100, 16383])
def test_workspace_bytes_ragged(dtype, esize, T):
    # a length that is not a multiple of 64 runs at the padded length, plus
    # zero-padded staging of q, k, v, w, out (d * esize per token) and beta,
    # logf, lse (4 bytes per token each)
    B, H, d = 2, 3, 64
    Tp = (T + 63) // 64 * 64
    base = pa.path_attn_workspace_bytes(B, H, Tp, d, dtype)
    n = pa.path_attn_workspace_bytes(B, H, T, d, dtype)
    if T == Tp:
        assert n == base
    else:
        rows = B * H * Tp
        expect = base + 5 * rows * d * esize + 3 * rows * 4
        assert expect <= n <= expect + 8 * 256


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=FAKE,
             B=1, H=2, T=256, d=64, dtype=pa.BF16, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.path_attn_fwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"], a["out"],
                             a["lse"], a["B"], a["H"], a["T"], a["d"], a["dtype"], a["ws"],
                             a["wsb"], a["stream"])


# every case below is invalid: validation rejects it before any HIP call
BAD_FWD = [
    (dict(q=None), EINVAL), (dict(k=None), EINVAL), (dict(v=None), EINVAL),
    (dict(w=None), EINVAL), (dict(beta=None), EINVAL), (dict(out=None), EINVAL),
    (dict(lse=None), EINVAL), (dict(ws=None), EINVAL),
    (dict(q=FAKE + 2), EINVAL), (dict(beta=FAKE + 4), EINVAL), (dict(out=FAKE + 8), EINVAL),
    (dict(logf=FAKE + 4), EINVAL), (dict(ws=FAKE + 16), EINVAL),
    (dict(wsb=1000), EINVAL), (dict(dtype=5), EINVAL), (dict(B=0), EINVAL),
    (dict(H=-1), EINVAL), (dict(T=0), EINVAL),
    (dict(d=96), EUNSUP), (dict(d=32), EUNSUP),
    (dict(B=1 << 12, H=1 << 10, T=1024), EUNSUP),
    (dict(T=200, wsb=1000), EINVAL),   # a ragged length still needs its staging
]


@pytest.mark.parametrize("kw,status", BAD_FWD, ids=lambda x: str(x))
def test_fwd_validation(kw, status):
    assert _fwd(pa.load_library(), **kw) == status


@pytest.mark.parametrize("scale,flags,status", [
    (-1.0, 0, EINVAL), (float("inf"), 0, EINVAL), (float("nan"), 0, EINVAL),
    (0.5, 4, EINVAL), (0.5, 0xFFFF, EINVAL)])
def test_fwd_ex_validation(scale, flags, status):
    # every case is invalid, so nothing is launched on the fake addresses
    lib = pa.load_library()
    assert lib.path_attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 2, 256, 64,
                                pa.BF16, scale, flags, FAKE, 1 << 40, None) == status


def test_prepare_and_stream_validation():
    lib = pa.load_library()
    assert lib.path_attn_prepare(FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 64, 64, 1, FAKE,
                                 1 << 40, None) == EINVAL
    assert lib.path_attn_prepare(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 64, 1, FAKE,
                                 10, None) == EINVAL
    assert lib.path_attn_prepare(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 96, 96, 1, FAKE,
                                 1 << 40, None) == EUNSUP
    # stream: bad use_gate, null out, misaligned lse, small workspace, bad d
    assert lib.path_attn_stream(FAKE, 1 << 40, 2, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert lib.path_attn_stream(FAKE, 1 << 40, 0, None, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert lib.path_attn_stream(FAKE, 1 << 40, 0, FAKE, FAKE + 4, 1, 1, 64, 64, 1, None) == EINVAL
    assert lib.path_attn_stream(FAKE, 100, 0, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert lib.path_attn_stream(FAKE, 1 << 40, 0, FAKE, FAKE, 1, 1, 64, 48, 1, None) == EUNSUP
    # stream_ex: unknown flag bits, misaligned counter, plus the stream checks
    ex = lib.path_attn_stream_ex
    assert ex(FAKE, 1 << 40, 1, 0.0, 2, None, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert ex(FAKE, 1 << 40, 1, 0.0, 1, FAKE + 4, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert ex(FAKE, 1 << 40, 2, 0.0, 0, None, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert ex(FAKE, 100, 1, 0.0, 0, None, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL
    assert ex(FAKE, 1 << 40, 1, 0.0, 1, None, FAKE, FAKE, 1, 1, 64, 48, 1, None) == EUNSUP
    assert ex(FAKE, 1 << 40, 1, -2.0, 0, None, FAKE, FAKE, 1, 1, 64, 64, 1, None) == EINVAL


def test_chunk_prep_validation():
    lib = pa.load_library()
    common = [FAKE, FAKE, FAKE, FAKE, FAKE, None]
    outs = [FAKE, FAKE, FAKE, FAKE, None]
    # misaligned optional output
    assert lib.path_attn_chunk_prep(*common, FAKE + 4, *outs[1:], 1, 1, 64, 64, 1, FAKE, 1 << 40, None) == EINVAL
    # workspace too small
    assert lib.path_attn_chunk_prep(*common, *outs, 1, 1, 64, 64, 1, FAKE, 10, None) == EINVAL
    # unsupported head dim
    assert lib.path_attn_chunk_prep(*common, *outs, 1, 1, 64, 80, 1, FAKE, 1 << 40, None) == EUNSUP
    # the unpack needs whole chunks
    assert lib.path_attn_chunk_prep(*common, *outs, 1, 1, 100, 64, 1, FAKE, 1 << 40, None) == EUNSUP


# ---- decoding entry points

def test_decode_workspace_sizes():
    # prefill: float32 ->K rows and per-chunk d x d transforms
    B, H, L, d = 2, 16, 16384, 64
    n = pa.load_library().path_attn_prefill_workspace_bytes(B, H, L, d)
    expect = B * H * L * d * 4 + B * H * (L // 64) * d * d * 4
    assert expect <= n <= expect + 512
    assert pa.load_library().path_attn_prefill_workspace_bytes(1, 1, 100, 64) == 0
    assert pa.load_library().path_attn_prefill_workspace_bytes(1, 1, 64, 96) == 0
    # decode: one (max, sum, d values) partial per head and 512-key split
    n = pa.load_library().path_attn_decode_workspace_bytes(B, H, 16386, d)
    assert n >= B * H * 33 * (d + 2) * 4
    assert pa.load_library().path_attn_decode_workspace_bytes(1, 1, 0, 64) == 0


def _prefill(lib, **kw):
    a = dict(k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, kc=FAKE, vc=FAKE, gc=None,
             B=1, H=2, L=128, T_cap=256, d=64, dtype=pa.BF16, kc_dtype=pa.F32, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.path_attn_prefill_cache(a["k"], a["v"], a["w"], a["beta"], a["logf"], a["kc"],
                                       a["vc"], a["gc"], a["B"], a["H"], a["L"], a["T_cap"],
                                       a["d"], a["dtype"], a["kc_dtype"], a["ws"], a["wsb"],
                                       a["stream"])


BAD_PREFILL = [
    (dict(k=None), EINVAL), (dict(kc=None), EINVAL), (dict(vc=None), EINVAL),
    (dict(logf=FAKE), EINVAL),                       # a gate needs the gate cache
    (dict(k=FAKE + 2), EINVAL), (dict(gc=FAKE + 8, logf=FAKE), EINVAL),
    (dict(ws=None), EINVAL), (dict(ws=FAKE + 16), EINVAL), (dict(wsb=100), EINVAL),
    (dict(L=-64), EINVAL), (dict(L=512), EINVAL),    # longer than the cache
    (dict(kc_dtype=3), EINVAL), (dict(dtype=2), EINVAL), (dict(T_cap=0), EINVAL),
    (dict(L=100), EUNSUP), (dict(d=80), EUNSUP),
    (dict(B=1 << 12, H=1 << 9, T_cap=1 << 14), EUNSUP),
]


@pytest.mark.parametrize("kw,status", BAD_PREFILL, ids=lambda x: str(x))
def test_prefill_validation(kw, status):
    assert _prefill(pa.load_library(), **kw) == status


def test_prefill_empty_prompt_launches_nothing():
    # L = 0 is valid and does nothing (no HIP call is made: the addresses are fake)
    assert _prefill(pa.load_library(), L=0, k=None, v=None, w=None, beta=None, ws=None) == OK


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, kc=FAKE, vc=FAKE, gc=None,
             t=5, out=FAKE, lse=FAKE, B=1, H=2, T_cap=256, d=64, dtype=pa.BF16,
             kc_dtype=pa.F32, scale=0.0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.path_attn_decode_step(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"],
                                     a["kc"], a["vc"], a["gc"], a["t"], a["out"], a["lse"],
                                     a["B"], a["H"], a["T_cap"], a["d"], a["dtype"],
                                     a["kc_dtype"], a["scale"], a["ws"], a["wsb"], a["stream"])


BAD_DECODE = [
    (dict(q=None), EINVAL), (dict(w=None), EINVAL), (dict(beta=None), EINVAL),
    (dict(kc=None), EINVAL), (dict(out=None), EINVAL), (dict(lse=None), EINVAL),
    (dict(ws=None), EINVAL), (dict(logf=FAKE), EINVAL), (dict(lse=FAKE + 2), EINVAL),
    (dict(beta=FAKE + 1), EINVAL), (dict(q=FAKE + 4), EINVAL),
    (dict(ws=FAKE + 64), EINVAL), (dict(wsb=8), EINVAL),
    (dict(t=-1), EINVAL), (dict(t=256), EINVAL), (dict(kc_dtype=-1), EINVAL),
    (dict(d=32), EUNSUP), (dict(B=1 << 12, H=1 << 9, T_cap=1 << 14), EUNSUP),
    (dict(scale=-1.0), EINVAL),
]


@pytest.mark.parametrize("kw,status", BAD_DECODE, ids=lambda x: str(x))
def test_decode_validation(kw, status):
    assert _decode(pa.load_library(), **kw) == status


def test_binding_has_no_cpu_fallback():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    b = torch.zeros(1, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        pa.path_attn_fwd(x, x, x, x, b)


def test_binding_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setenv("PATH_ATTN_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not found"):
        binding.load_library()


# ---- backward

@pytest.mark.parametrize("dtype,esize", [(pa.F32, 4), (pa.BF16, 2)])
@pytest.mark.parametrize("B,H,T,d", [(2, 16, 2048, 64), (1, 2, 256, 128)])
def test_bwd_workspace_bytes(dtype, esize, B, H, T, d):
    lib = pa.load_library()
    n = lib.path_attn_bwd_workspace_bytes(B, H, T, d, dtype)
    BH, N = B * H, T // 64
    # key levels (input dtype), dM partials per key-chunk group
    G = (4 if d == 64 else 2) if dtype == pa.BF16 else (2 if d == 64 else 1)
    copies = 1 if (dtype == pa.BF16 and d == 64) else 2   # rows, and transposed where needed
    big = copies * BH * N * (N - 1) // 2 * 64 * d * esize + BH * N * ((N + G - 1) // G) * d * d * 4
    # plus per-token and per-chunk arrays
    assert big < n < big + BH * T * d * 4 * 24 + BH * N * (d * d + 64 * 64) * 4 * 16
    # a ragged length runs at the next multiple of 64 plus staging rows
    assert lib.path_attn_bwd_workspace_bytes(1, 1, 100, 64, pa.F32) > lib.path_attn_bwd_workspace_bytes(1, 1, 128, 64, pa.F32)
    assert lib.path_attn_bwd_workspace_bytes(1, 1, 64, 96, pa.F32) == 0
    assert lib.path_attn_bwd_workspace_bytes(1, 1, 64, 64, 4) == 0


@pytest.mark.parametrize("dtype", [pa.F32, pa.BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_workspace_windows(dtype, d):
    """Past 33 chunks the default backward sweep runs in windows of 16 query
    chunks: its workspace grows as about T^1.5 instead of T^2, and longer
    windows (window_bytes) cost more, up to the single window that stores
    every key level."""
    lib = pa.load_library()
    nb = lambda T: lib.path_attn_bwd_workspace_bytes(1, 4, T, d, dtype)
    nw = lambda T, w: lib.path_attn_bwd_workspace_bytes_window(1, 4, T, d, dtype, w)
    # up to 33 chunks: one window by default
    for T in (64, 1024, 2112):
        assert nb(T) == nw(T, 0) == nw(T, 10 ** 6)
    # 65 chunks and more: windows of 16 by default, longer windows cost more
    for T in (4160, 8192, 16384):
        assert nb(T) == nw(T, 16) < nw(T, 32) < nw(T, 64) <= nw(T, 0)
    # the quadratic term is gone: doubling T at most triples the workspace
    # (it quadruples with one window)
    assert nb(32768) < 3.0 * nb(16384)
    assert nw(32768, 0) > 3.5 * nw(16384, 0)
    # the benchmark shape: 18.19 GiB with one window (the saved per-chunk
    # matrices in bytes of their own), under 4 GiB by default
    big = lib.path_attn_bwd_workspace_bytes_window(2, 16, 16384, 64, pa.BF16, 0)
    small = lib.path_attn_bwd_workspace_bytes(2, 16, 16384, 64, pa.BF16)
    assert abs(big / 2 ** 30 - 18.19) < 0.01 and small / 2 ** 30 < 4.0
    assert lib.path_attn_bwd_workspace_bytes_window(1, 1, 64, 96, pa.F32, 16) == 0


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=FAKE,
             dout=FAKE, dlse=None, dq=FAKE, dk=FAKE, dv=FAKE, dw=FAKE, dbeta=FAKE, dlogf=None,
             B=1, H=2, T=256, d=64, dtype=pa.BF16, scale=0.0, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return lib.path_attn_bwd(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"], a["out"],
                             a["lse"], a["dout"], a["dlse"], a["dq"], a["dk"], a["dv"], a["dw"],
                             a["dbeta"], a["dlogf"], a["B"], a["H"], a["T"], a["d"], a["dtype"],
                             a["scale"], a["ws"], a["wsb"], a["stream"])


# every case fails validation (the addresses are fake and must never be launched on)
BAD_BWD = [
    (dict(q=None), EINVAL), (dict(v=None), EINVAL), (dict(out=None), EINVAL),
    (dict(lse=None), EINVAL), (dict(dout=None), EINVAL), (dict(dq=None), EINVAL),
    (dict(dw=None), EINVAL), (dict(dbeta=None), EINVAL), (dict(ws=None), EINVAL),
    (dict(logf=FAKE), EINVAL),                      # the gate needs dlogf
    (dict(q=FAKE + 4), EINVAL), (dict(dlse=FAKE + 4), EINVAL), (dict(dbeta=FAKE + 8), EINVAL),
    (dict(logf=FAKE, dlogf=FAKE + 2), EINVAL),
    (dict(ws=FAKE + 64), EINVAL), (dict(wsb=100), EINVAL),
    (dict(scale=-1.0), EINVAL), (dict(scale=float("nan")), EINVAL), (dict(dtype=5), EINVAL),
    (dict(T=100, wsb=100), EINVAL), (dict(T=0), EINVAL), (dict(d=96), EUNSUP), (dict(B=0), EINVAL),
    (dict(B=1 << 12, H=1 << 9, T=1 << 14), EUNSUP),
]


@pytest.mark.parametrize("kw,status", BAD_BWD, ids=lambda x: str(x))
def test_bwd_validation(kw, status):
    assert _bwd(pa.load_library(), **kw) == status


# ---- strided and packed batches

def test_varlen_workspace_bytes():
    lib = pa.load_library()
    for dt, e in ((pa.F32, 4), (pa.BF16, 2)):
        # views are always staged: the dense layout plus 4 vector and 4 scalar staging arrays
        dense = pa.path_attn_workspace_bytes(2, 3, 128, 64, dt)
        n = pa.path_attn_varlen_workspace_bytes(2, 3, 128, 64, dt)
        assert n >= dense + 6 * 128 * (5 * 64 * e + 3 * 4)
        # a ragged dense call stages too, with the same layout
        assert pa.path_attn_varlen_workspace_bytes(2, 3, 100, 64, dt) == \
            pa.path_attn_workspace_bytes(2, 3, 100, 64, dt)
        nb = lib.path_attn_bwd_varlen_workspace_bytes(2, 3, 128, 64, dt)
        assert nb >= lib.path_attn_bwd_workspace_bytes(2, 3, 128, 64, dt) + \
            6 * 128 * (10 * 64 * e + 6 * 4)
        assert lib.path_attn_bwd_varlen_workspace_bytes(2, 3, 100, 64, dt) == \
            lib.path_attn_bwd_workspace_bytes(2, 3, 100, 64, dt)
    assert pa.path_attn_varlen_workspace_bytes(1, 1, 64, 80, pa.F32) == 0
    assert lib.path_attn_bwd_varlen_workspace_bytes(0, 1, 64, 64, pa.F32) == 0


def _dense_strides(n, H, T, d):
    return [(H * T * d, T * d, d)] * n


def _fwd_varlen(lib, strides=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=FAKE,
             cu=None, B=1, H=2, T=256, d=64, dtype=pa.BF16, scale=0.0, flags=0, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    if strides is None:
        strides = _dense_strides(5, a["H"], a["T"], a["d"]) + _dense_strides(3, a["H"], a["T"], 1)
    arr = None if strides == "null" else binding._stride_array(strides)
    return lib.path_attn_fwd_varlen(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"],
                                    a["out"], a["lse"], arr, a["cu"], a["B"], a["H"], a["T"],
                                    a["d"], a["dtype"], a["scale"], a["flags"], a["ws"], a["wsb"],
                                    a["stream"])


def _with(strides_index, value, n_vec=5, n=8):
    st = _dense_strides(n_vec, 2, 256, 64) + _dense_strides(n - n_vec, 2, 256, 1)
    st[strides_index] = value
    return st


# every case fails validation (fake addresses, never launched on)
BAD_FWD_VARLEN = [
    (dict(strides="null"), EINVAL), (dict(q=None), EINVAL), (dict(out=None), EINVAL),
    (dict(lse=None), EINVAL), (dict(beta=None), EINVAL), (dict(ws=None), EINVAL),
    (dict(q=FAKE + 2), EINVAL), (dict(lse=FAKE + 2), EINVAL), (dict(cu=FAKE + 2), EINVAL),
    (dict(logf=FAKE + 1), EINVAL), (dict(ws=FAKE + 64), EINVAL), (dict(wsb=100), EINVAL),
    (dict(strides=_with(0, (-1, 64, 64))), EINVAL),        # negative stride
    (dict(strides=_with(2, (0, 64, 65))), EINVAL),         # odd bf16 stride: 2-byte rows
    (dict(strides=_with(4, (1 << 40, 64, 64))), EINVAL),   # stride too large
    (dict(strides=_with(6, (0, -4, 1)), logf=FAKE), EINVAL),
    (dict(scale=-1.0), EINVAL), (dict(flags=4), EINVAL), (dict(dtype=3), EINVAL),
    (dict(T=0), EINVAL), (dict(d=96), EUNSUP), (dict(B=1 << 12, H=1 << 9, T=1 << 14), EUNSUP),
]


@pytest.mark.parametrize("kw,status", BAD_FWD_VARLEN, ids=lambda x: str(x))
def test_fwd_varlen_validation(kw, status):
    assert _fwd_varlen(pa.load_library(), **kw) == status


def _bwd_varlen(lib, strides=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, beta=FAKE, logf=None, out=FAKE, lse=FAKE,
             dout=FAKE, dlse=None, dq=FAKE, dk=FAKE, dv=FAKE, dw=FAKE, dbeta=FAKE, dlogf=None,
             cu=None, B=1, H=2, T=256, d=64, dtype=pa.BF16, scale=0.0, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    if strides is None:
        strides = _dense_strides(10, a["H"], a["T"], a["d"]) + _dense_strides(6, a["H"], a["T"], 1)
    arr = None if strides == "null" else binding._stride_array(strides)
    return lib.path_attn_bwd_varlen(a["q"], a["k"], a["v"], a["w"], a["beta"], a["logf"],
                                    a["out"], a["lse"], a["dout"], a["dlse"], a["dq"], a["dk"],
                                    a["dv"], a["dw"], a["dbeta"], a["dlogf"], arr, a["cu"],
                                    a["B"], a["H"], a["T"], a["d"], a["dtype"], a["scale"],
                                    a["ws"], a["wsb"], a["stream"])


BAD_BWD_VARLEN = [
    (dict(strides="null"), EINVAL), (dict(dout=None), EINVAL), (dict(dq=None), EINVAL),
    (dict(dbeta=None), EINVAL), (dict(logf=FAKE), EINVAL),   # the gate needs dlogf
    (dict(dk=FAKE + 2), EINVAL), (dict(dlse=FAKE + 1), EINVAL), (dict(cu=FAKE + 1), EINVAL),
    (dict(wsb=100), EINVAL), (dict(ws=FAKE + 32), EINVAL), (dict(scale=float("inf")), EINVAL),
    (dict(strides=_with(7, (0, 64, 63), n_vec=10, n=16)), EINVAL),
    (dict(strides=_with(13, (-1, 0, 1), n_vec=10, n=16), dlse=FAKE), EINVAL),
    (dict(T=0), EINVAL), (dict(d=32), EUNSUP), (dict(dtype=-1), EINVAL),
]


@pytest.mark.parametrize("kw,status", BAD_BWD_VARLEN, ids=lambda x: str(x))
def test_bwd_varlen_validation(kw, status):
    assert _bwd_varlen(pa.load_library(), **kw) == status


def test_varlen_binding_needs_gpu_tensors():
    import torch
    x = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError, match="GPU"):
        pa.path_attn_fwd_varlen(x, x, x, x, torch.zeros(1, 2, 64))
    with pytest.raises(ValueError, match="GPU"):
        pa.path_attn_bwd_varlen(x, x, x, x, torch.zeros(1, 2, 64), None, x, None, x)


@pytest.mark.parametrize("B,H,T,d,dtype,null_q,scale,flags,status", [
    (1, 16, 8192, 64, pa.BF16, False, 0.0, 0, EINVAL),   # workspace above the fixed array
    (1, 8, 8192, 128, pa.BF16, False, 0.0, 0, EINVAL),
    (1, 2, 256, 64, pa.BF16, True, 0.0, 0, EINVAL),      # null q
    (1, 2, 256, 64, pa.BF16, False, -1.0, 0, EINVAL),    # bad scale
    (1, 2, 256, 64, pa.BF16, False, 0.0, 4, EINVAL),     # unknown flag
    (1, 2, 256, 96, pa.BF16, False, 0.0, 0, EUNSUP),
])
def test_noalloc_validation(B, H, T, d, dtype, null_q, scale, flags, status):
    """path_attn_fwd_noalloc checks its arguments, the problem size against
    the fixed array included, before any HIP call."""
    assert pa.path_attn_workspace_bytes(1, 16, 4096, 64, pa.BF16) <= pa.NOALLOC_MAX_BYTES
    lib = pa.load_library()
    q = None if null_q else FAKE
    assert lib.path_attn_fwd_noalloc(q, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, B, H, T, d,
                                     dtype, scale, flags, None) == status


def test_noalloc_max_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PATH_ATTN_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pa.NOALLOC_MAX_BYTES


@pytest.mark.parametrize("d,d_path,status", [(64, 48, EUNSUP), (128, 96, EUNSUP), (64, 0, EINVAL),
                                             (64, 80, EINVAL), (128, -64, EINVAL)])
def test_partial_validation(d, d_path, status):
    """path_attn_fwd_partial: d_path must be d or d / 2 (EUNSUPPORTED for other
    values in (0, d], EINVAL outside), checked before any HIP call."""
    lib = pa.load_library()
    assert lib.path_attn_fwd_partial(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 2, 256, d,
                                     d_path, pa.BF16, 0.0, 0, FAKE, 1 << 40, None) == status


def test_partial_workspace_fits_the_full_one():
    """A workspace of path_attn_workspace_bytes suffices for partial PaTH: a
    smaller one is rejected only below the partial layout's own size."""
    lib = pa.load_library()
    need = pa.path_attn_workspace_bytes(1, 2, 256, 64, pa.BF16)
    assert lib.path_attn_fwd_partial(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 2, 256, 64,
                                     32, pa.BF16, 0.0, 0, FAKE, 100, None) == EINVAL
    assert need > 100


def test_wbeta_validation():
    """path_attn_wbeta rejects bad arguments before any HIP call: every call
    below has exactly one invalid argument (the pointers are aligned
    stand-ins, never dereferenced)."""
    lib = pa.load_library()
    P = 1 << 20

    def call(x=P, wd=P, wu=P, cw=P, u=P, ub=P, w=P, beta=P, B=1, T=64, Dm=64, R=32, H=2, d=64,
             dtype=pa.BF16):
        return lib.path_attn_wbeta(x, wd, wu, cw, u, ub, w, beta, B, T, Dm, R, H, d, dtype, None)

    for name in ("x", "wd", "wu", "cw", "u", "ub", "w", "beta"):
        assert call(**{name: None}) == EINVAL, name
    for name in ("x", "wd", "wu", "cw", "u", "w"):
        assert call(**{name: P + 8}) == EINVAL, name   # 16-byte loads and stores
    assert call(ub=P + 2) == EINVAL and call(beta=P + 2) == EINVAL
    for kw in ({"B": 0}, {"T": 0}, {"Dm": 0}, {"R": 0}, {"H": 0}, {"d": 0}, {"dtype": 7}):
        assert call(**kw) == EINVAL, kw
    for kw in ({"dtype": pa.F32}, {"d": 96}, {"Dm": 40}, {"Dm": 96}, {"R": 24}, {"R": 144}):
        assert call(**kw) == EUNSUP, kw
