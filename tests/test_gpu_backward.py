"""GPU parity of the backward pass (path_attn_bwd) against the float64
gradient oracles.

The forward runs on the GPU (path_attn_fwd) and its out and lse feed the
GPU backward, as a training step would use them.  The oracle recomputes
everything in float64 from the same stored inputs and cotangents.

  * Small cases (several chunks, d = 64 and 128, with and without the gate,
    with and without a gradient on lse, and lengths that are not a multiple
    of 64): every gradient of every head against oracle.backward.gradients
    (autograd of the definition).
  * The workloads at full size: sampled heads against
    oracle.chunked_backward.sweep_backward (the blockwise float64 statement,
    pinned to the autograd oracle on the CPU), the GPU run covering the whole
    batch in the same launch configuration as any other call.

Bar, per gradient tensor g with float64 reference r:
    max |g - r| <= tol * max(1, max |r|)
with tol = 2e-4 for float32 inputs (float32 arithmetic; the longest sums
run over T keys or T queries, sqrt(T) * 2^-24 ~ 1e-6 typical, plus the
float32 forward's out and lse) and tol = 2e-2 for bf16 inputs (the forward's
out is rounded to bf16, 2^-9 relative, which enters rowdot(dout, out) and so
every softmax gradient; each gradient is rounded to bf16 once more on
output).  dlogf at position 0 must be exactly zero (f_0 enters no logit).
"""
from __future__ import annotations

import time

import numpy as np
import pytest

import workloads
from oracle.backward import gradients as oracle_gradients
from oracle.chunked_backward import sweep_backward
from tests.gpu_util import record, spread_heads, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")


def _log(msg):
    print(msg, flush=True)


def _to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _run_gpu(inp, cot, dtype, scale=None):
    import torch
    import householder_position_encoding_amd as pa
    dev = to_device(inp, dtype)
    tdt = dev["q"].dtype
    dout = torch.from_numpy(cot["dout"]).to(device="cuda", dtype=tdt).contiguous()
    dlse = None if cot["dlse"] is None else torch.from_numpy(cot["dlse"]).cuda().contiguous()
    out, lse = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"],
                                scale=scale)
    grads = pa.path_attn_bwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"],
                             out, lse, dout, dlse, scale=scale)
    torch.cuda.synchronize()
    return {n: (None if g is None else _to_np(g)) for n, g in zip(NAMES, grads)}


def _head(inp, cot, b, h):
    sel = lambda x: None if x is None else np.asarray(x[b, h], dtype=np.float64)
    return (sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["w"]), sel(inp["beta"]),
            sel(inp["logf"]), sel(cot["dout"]), sel(cot["dlse"]))


def _compare(tag, dtype, got, ref, b, h):
    tol = TOL[dtype]
    errs = {}
    for n in NAMES:
        r = ref[n]
        if r is None:
            assert got[n] is None, f"{tag}: {n} returned without the gate"
            continue
        g = got[n][b, h]
        assert np.all(np.isfinite(g)), f"{tag}: {n} not finite"
        scale = max(1.0, float(np.max(np.abs(r))))
        errs[n] = float(np.max(np.abs(g - r))) / scale
    # max|g - r| / max(1, max|r|) per gradient
    record(f"backward {tag} head ({b},{h})", tol=tol, **{f"err_{n}": e for n, e in errs.items()})
    for n, err in errs.items():
        assert err <= tol, f"{tag}: {n} of head ({b},{h}) off by {err:.3g} > {tol}"
    if ref["dlogf"] is not None:
        assert got["dlogf"][b, h, 0] == 0.0
    return max(errs.values())


SMALL = [
    # dtype, d, fox, dlse, B, H, T
    ("f32", 64, False, False, 1, 2, 256),
    ("f32", 64, True, True, 1, 2, 256),
    ("f32", 128, True, True, 2, 1, 192),
    ("f32", 64, False, True, 1, 1, 64),
    ("f32", 128, False, False, 1, 1, 128),
    ("bf16", 64, True, True, 1, 2, 256),
    ("bf16", 128, False, True, 1, 2, 192),
    ("bf16", 64, False, False, 2, 1, 320),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_backward_small_all_heads(case):
    dtype, d, fox, with_dlse, B, H, T = case
    _log(f"backward small {case}")
    inp = workloads.small(dtype, B, H, T, d, seed=70 + T + d, fox=fox, beta_sigma=1.5)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=170 + T + d, with_dlse=with_dlse)
    got = _run_gpu(inp, cot, dtype)
    for b in range(B):
        for h in range(H):
            ref = oracle_gradients(*_head(inp, cot, b, h))
            _compare(f"small {case}", dtype, got, ref, b, h)


RAGGED = [
    # dtype, d, fox, dlse, B, H, T
    ("f32", 64, True, True, 1, 2, 1),
    ("f32", 64, False, True, 1, 1, 63),
    ("f32", 128, True, False, 1, 1, 100),
    ("bf16", 64, True, True, 2, 1, 130),
    ("bf16", 128, False, True, 1, 2, 65),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_backward_ragged_length(case):
    """Lengths that are not a multiple of 64: every gradient of every head
    against the oracle on the unpadded sequence."""
    dtype, d, fox, with_dlse, B, H, T = case
    _log(f"backward ragged {case}")
    inp = workloads.small(dtype, B, H, T, d, seed=80 + T + d, fox=fox, beta_sigma=1.5)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=180 + T + d, with_dlse=with_dlse)
    got = _run_gpu(inp, cot, dtype)
    assert got["dq"].shape == (B, H, T, d) and got["dbeta"].shape == (B, H, T)
    for b in range(B):
        for h in range(H):
            ref = oracle_gradients(*_head(inp, cot, b, h))
            _compare(f"ragged {case}", dtype, got, ref, b, h)


def test_backward_custom_scale_and_near_reflections():
    """An explicit softmax scale, and betas close to 2 (near reflections)."""
    dtype, d, B, H, T = "f32", 64, 1, 2, 256
    inp = workloads.small(dtype, B, H, T, d, seed=91, fox=True, near2_frac=0.3)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=191)
    got = _run_gpu(inp, cot, dtype, scale=0.3)
    for h in range(H):
        q, k, v, w, beta, logf, do, dl = _head(inp, cot, 0, h)
        ref = oracle_gradients(q, k, v, w, beta, logf, do, dl, scale=0.3)
        _compare("scale 0.3, near-2 betas", dtype, got, ref, 0, h)


# Heads compared at full size: spread over the flat head index where the
# blockwise oracle is cheap (T = 2048: about 1 s a head), fewer at T = 8192
# and 16384 (about 20 and 45 s a head on the CPU).
FULL = [
    (workloads.MID_D64, spread_heads(16, 16)),
    (workloads.MID_D128_NEAR2, [(0, 0), (5, 3), (10, 6), (15, 7)]),
    (workloads.FOX_D128, [(1, 2), (3, 7)]),
    (workloads.LONG_D64, [(1, 15)]),
]


@pytest.mark.parametrize("wl,heads", FULL, ids=lambda x: getattr(x, "name", "heads"))
def test_backward_full_size_sampled_heads(wl, heads):
    _log(f"backward full size {wl.name}: generating inputs")
    inp = workloads.generate(wl)
    cot = workloads.cotangents(wl.dtype, wl.B, wl.H, wl.T, wl.d, seed=1000 + wl.seed)
    t0 = time.time()
    got = _run_gpu(inp, cot, wl.dtype)
    _log(f"{wl.name}: GPU forward + backward done in {time.time() - t0:.1f} s")
    for b, h in heads:
        q, k, v, w, beta, logf, do, dl = _head(inp, cot, b, h)
        import oracle
        o, lse = oracle.path_attn(q, k, v, w, beta, logf)
        t0 = time.time()
        ref = sweep_backward(q, k, v, w, beta, logf, do, o, lse, dlse=dl)
        _log(f"{wl.name}: oracle head ({b},{h}) in {time.time() - t0:.1f} s")
        _compare(wl.name, wl.dtype, got, ref, b, h)


def test_backward_fox_d64_medium():
    """bf16, d = 64, with the gate, at T = 2048 (32 chunks): the level walk,
    dq64 and dk64 run their steady loops (warm-up levels, unrolled step pairs,
    gate values fetched with the level rows), which the small cases are too
    short to reach; one head against the blockwise float64 oracle."""
    B, H, T, d = 1, 2, 2048, 64
    inp = workloads.small("bf16", B, H, T, d, seed=2048 + 64, fox=True)
    cot = workloads.cotangents("bf16", B, H, T, d, seed=3072)
    got = _run_gpu(inp, cot, "bf16")
    q, k, v, w, beta, logf, do, dl = _head(inp, cot, 0, 1)
    import oracle
    o, lse = oracle.path_attn(q, k, v, w, beta, logf)
    t0 = time.time()
    ref = sweep_backward(q, k, v, w, beta, logf, do, o, lse, dlse=dl)
    _log(f"fox d64 T={T}: oracle head (0,1) in {time.time() - t0:.1f} s")
    _compare("fox d64 medium", "bf16", got, ref, 0, 1)


# Past 33 chunks the sweep runs in windows of 16 query chunks: a float32
# checkpoint pass of the level walk, then per window (the last first) its own
# levels, dq, dk (Gamma handed to the window below through the workspace) and
# the dM reduction.  T = 4160 is 65 chunks (windows [1, 17), [17, 33),
# [33, 49), [49, 65)); T = 2176 is 34 chunks, whose last window holds one
# query chunk.  One head each against the blockwise oracle.
WINDOWED = [
    # dtype, d, fox, B, H, T, head
    ("bf16", 64, True, 1, 2, 4160, (0, 1)),
    ("bf16", 128, False, 1, 1, 2176, (0, 0)),
    ("bf16", 128, True, 1, 1, 4160, (0, 0)),
    ("f32", 64, True, 1, 1, 4160, (0, 0)),
    ("f32", 128, False, 1, 1, 2176, (0, 0)),
]


@pytest.mark.parametrize("case", WINDOWED, ids=lambda c: "-".join(map(str, c[:6])))
def test_backward_windowed_sweep(case):
    dtype, d, fox, B, H, T, (b, h) = case
    inp = workloads.small(dtype, B, H, T, d, seed=4096 + d + T, fox=fox)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=5120 + T)
    got = _run_gpu(inp, cot, dtype)
    q, k, v, w, beta, logf, do, dl = _head(inp, cot, b, h)
    import oracle
    o, lse = oracle.path_attn(q, k, v, w, beta, logf)
    t0 = time.time()
    ref = sweep_backward(q, k, v, w, beta, logf, do, o, lse, dlse=dl)
    _log(f"windowed {dtype} d{d} T={T}: oracle head ({b},{h}) in {time.time() - t0:.1f} s")
    _compare(f"windowed {dtype} d{d} T={T}", dtype, got, ref, b, h)


@pytest.mark.parametrize("T,window", [(8192, None), (4160, 0)])
def test_backward_fox_skip_is_exact(T, window):
    """bf16, d = 128, with the gate: the backward leaves out every block of 32
    keys and a query chunk whose weights are exactly zero (path_attn_bwd_ex
    without PATH_ATTN_NO_SKIP).  The gradients must be the same bits as with
    every block computed, in the windowed sweep and with one window; the
    decaying gate of the FoX workload makes most far blocks vanish."""
    import torch
    import householder_position_encoding_amd as pa
    B, H, d = 1, 2, 128
    inp = workloads.small("bf16", B, H, T, d, seed=8192 + T, fox=True)
    cot = workloads.cotangents("bf16", B, H, T, d, seed=9000 + T)
    dev = to_device(inp, "bf16")
    dout = torch.from_numpy(cot["dout"]).to(device="cuda", dtype=torch.bfloat16).contiguous()
    dlse = torch.from_numpy(cot["dlse"]).cuda().contiguous()
    out, lse = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"])
    args = (dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"], out, lse, dout, dlse)
    code = 1
    need = (pa.path_attn_bwd_workspace_bytes(B, H, T, d, code) if window is None
            else pa.path_attn_bwd_workspace_bytes_window(B, H, T, d, code, window))

    def nan_workspace():
        # every byte 0xFF (a NaN in bf16 and float32): a read of anything the
        # call did not write shows in the gradients
        return torch.full((need,), 255, dtype=torch.uint8, device="cuda")

    g_skip = pa.path_attn_bwd(*args, window=window, workspace=nan_workspace())
    g_full = pa.path_attn_bwd(*args, window=window, flags=pa.NO_SKIP, workspace=nan_workspace())
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, g_skip, g_full):
        assert torch.equal(a.float(), b.float()), f"{name} differs with the skip"
    # every sum of the backward is taken in a fixed order: a second call
    # gives the same bits
    g_again = pa.path_attn_bwd(*args, window=window, workspace=nan_workspace())
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, g_again, g_skip):
        assert torch.equal(a.float(), b.float()), f"{name} differs between two calls"
