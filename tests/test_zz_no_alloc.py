"""path_attn_fwd_noalloc (the forward whose workspace is the library's fixed
device array) against path_attn_fwd_ex with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller (ragged) problem, so the
array holds the first call's contents when the second runs; results must be
the same bits, and within the parity bar of the fp64 oracle."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_util import TOL, oracle_full, to_device

pytestmark = pytest.mark.gpu


def _lib():
    import householder_position_encoding_amd as pa
    lib = ctypes.CDLL(pa.library_path())
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.path_attn_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.path_attn_workspace_bytes.restype = sz
    lib.path_attn_fwd_ex.argtypes = [vp] * 8 + [ci] * 5 + [ctypes.c_float, ctypes.c_uint, vp, sz, vp]
    lib.path_attn_fwd_ex.restype = ci
    lib.path_attn_fwd_noalloc.argtypes = [vp] * 8 + [ci] * 5 + [ctypes.c_float, ctypes.c_uint, vp]
    lib.path_attn_fwd_noalloc.restype = ci
    return lib


def _run_both(lib, dtype, B, H, T, d, fox, seed):
    import torch
    inp = workloads.small(dtype, B, H, T, d, seed=seed, fox=fox)
    dev = to_device(inp, dtype)
    code = 1 if dtype == "bf16" else 0
    stream = torch.cuda.current_stream().cuda_stream
    args = [dev[n].data_ptr() for n in ("q", "k", "v", "w", "beta")]
    args.append(dev["logf"].data_ptr() if fox else None)
    outs = []
    for noalloc in (True, False):
        out = torch.full_like(dev["q"], float("nan"))
        lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = lib.path_attn_fwd_noalloc(*args, out.data_ptr(), lse.data_ptr(), B, H, T, d,
                                           code, 0.0, 0, stream)
        else:
            nbytes = lib.path_attn_workspace_bytes(B, H, T, d, code)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            st = lib.path_attn_fwd_ex(*args, out.data_ptr(), lse.data_ptr(), B, H, T, d, code,
                                      0.0, 0, ws.data_ptr(), nbytes, stream)
        assert st == 0, (noalloc, st)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return inp, outs


@pytest.mark.parametrize("dtype,d,fox", [("bf16", 64, False), ("bf16", 128, True), ("f32", 64, True)])
def test_noalloc_matches_workspace_entry_point(dtype, d, fox):
    import torch
    lib = _lib()
    for (B, H, T, seed) in ((2, 4, 1024, 301), (1, 2, 200, 302)):   # second: smaller, ragged
        print(f"noalloc {dtype} d={d} fox={fox} B={B} H={H} T={T}", flush=True)
        inp, ((o_n, l_n), (o_w, l_w)) = _run_both(lib, dtype, B, H, T, d, fox, seed)
        ibits = torch.int16 if dtype == "bf16" else torch.int32
        assert torch.equal(o_n.view(ibits), o_w.view(ibits))
        assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32))
        o_ref, l_ref = oracle_full(inp)
        tol_o, tol_l = TOL[dtype]
        eo = float(np.max(np.abs(o_n.float().cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(l_n.cpu().numpy() - l_ref)))
        print(f"  max|do|={eo:.3g} max|dlse|={el:.3g}", flush=True)
        assert eo <= tol_o and el <= tol_l


def test_noalloc_rejects_a_problem_above_the_array():
    """B*H*T beyond the fixed array is EINVAL, checked before any HIP call;
    the largest bf16 d = 64 problem of 16 heads that fits runs."""
    import torch
    import householder_position_encoding_amd as pa
    lib = _lib()
    assert pa.path_attn_workspace_bytes(1, 16, 8192, 64, 1) > pa.NOALLOC_MAX_BYTES
    x = torch.zeros((1, 16, 8192, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((1, 16, 8192), dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    st = lib.path_attn_fwd_noalloc(p, p, p, p, b.data_ptr(), None, p, b.data_ptr(), 1, 16, 8192,
                                   64, 1, 0.0, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 1
    assert pa.path_attn_workspace_bytes(1, 16, 4096, 64, 1) <= pa.NOALLOC_MAX_BYTES
    inp = workloads.small("bf16", 1, 16, 4096, 64, seed=303)
    dev = to_device(inp, "bf16")
    out, lse = pa.path_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"])
    ref_o, ref_l = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
