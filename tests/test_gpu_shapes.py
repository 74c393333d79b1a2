"""GPU parity for general shapes: sequence lengths that are not a multiple of
the 64-token chunk, an explicit softmax scale, and partial PaTH (a direction
w_t that is zero on some coordinates, so those coordinates carry no position
transform).

Lengths are padded inside the library with identity factors (beta = 0,
w = 0) and zero q, k, v and gate; the padded tokens come after every real
token, so every real output must equal the oracle's on the unpadded
sequence.  Bars as in the forward parity tests: 1e-4 for float32 inputs; for
bf16 inputs 2e-2 on o and 1e-2 on lse.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, oracle_full, run_hip, to_device

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check(name, dtype, out, lse, o_ref, l_ref):
    tol_o, tol_l = TOL[dtype]
    eo = float(np.max(np.abs(out - o_ref)))
    el = float(np.max(np.abs(lse - l_ref)))
    _log(f"{name}: max|do|={eo:.3g} (tol {tol_o}) max|dlse|={el:.3g} (tol {tol_l})")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= tol_o and el <= tol_l


RAGGED = [
    # dtype, d, fox, B, H, T
    ("f32", 64, False, 1, 2, 1),
    ("f32", 64, True, 1, 2, 63),
    ("f32", 128, False, 2, 1, 65),
    ("bf16", 64, False, 2, 2, 100),
    ("bf16", 64, True, 1, 3, 300),
    ("bf16", 128, True, 1, 2, 130),
    ("f32", 128, True, 1, 1, 1000),
    ("bf16", 64, False, 1, 2, 1023),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "-".join(map(str, c)))
def test_ragged_length_all_rows(case):
    dtype, d, fox, B, H, T = case
    inp = workloads.small(dtype, B, H, T, d, seed=50 + T, fox=fox, beta_sigma=1.5)
    out, lse = run_hip(to_device(inp, dtype))
    assert out.shape == (B, H, T, d) and lse.shape == (B, H, T)
    o_ref, l_ref = oracle_full(inp)
    _check(f"ragged {case}", dtype, out, lse, o_ref, l_ref)


def test_ragged_prepare_then_stream_and_reuse():
    """The two-phase entry points on a ragged length give the same bits as the
    one-call forward, and a workspace reused for a second problem of the same
    shape gives that problem's result."""
    import torch
    import householder_position_encoding_amd as pa
    dtype, d, B, H, T = "bf16", 64, 1, 2, 200
    outs = []
    ws = None
    for seed in (3, 4):
        inp = workloads.small(dtype, B, H, T, d, seed=seed, fox=True)
        dev = to_device(inp, dtype)
        ws = pa.path_attn_prepare(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"],
                                  workspace=ws)
        out = torch.empty_like(dev["q"])
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        pa.path_attn_stream(ws, True, out, lse)
        o1, l1 = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"])
        torch.cuda.synchronize()
        assert torch.equal(out, o1) and torch.equal(lse, l1)
        o_ref, l_ref = oracle_full(inp)
        _check(f"prepare+stream seed {seed}", dtype, out.float().cpu().numpy().astype(np.float64),
               lse.cpu().numpy().astype(np.float64), o_ref, l_ref)
        outs.append(out)
    assert not torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("dtype,d,fox,scale", [("f32", 64, False, 0.3), ("f32", 128, True, 0.05),
                                               ("bf16", 64, False, 0.2), ("bf16", 128, True, 0.11)])
def test_custom_scale(dtype, d, fox, scale):
    import torch
    import householder_position_encoding_amd as pa
    B, H, T = 1, 2, 320
    inp = workloads.small(dtype, B, H, T, d, seed=61, fox=fox)
    dev = to_device(inp, dtype)
    out, lse = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"],
                                scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.path_attn(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"],
                                    inp["logf"], scale=scale)
    _check(f"scale {scale} {dtype} d={d} fox={fox}", dtype,
           out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
           o_ref, l_ref)


def test_decode_custom_scale():
    import torch
    import householder_position_encoding_amd as pa
    dtype, d, B, H, L, n_dec, scale = "f32", 64, 1, 2, 64, 5, 0.21
    inp = workloads.small(dtype, B, H, L + n_dec, d, seed=62)
    dev = to_device(inp, dtype)
    cache = pa.DecodeCache(B, H, L + n_dec, d, torch.float32)
    pa.path_attn_prefill_cache(cache, *(x[:, :, :L].contiguous() for x in (dev["k"], dev["v"], dev["w"], dev["beta"])))
    rows = np.stack([np.zeros(n_dec, dtype=np.int64), np.arange(L, L + n_dec)], 1)
    got_o, got_l = [], []
    for t in range(L, L + n_dec):
        at = lambda x: x[:, :, t].contiguous()
        o, l = pa.path_attn_decode_step(cache, at(dev["q"]), at(dev["k"]), at(dev["v"]), at(dev["w"]),
                                        at(dev["beta"]), scale=scale)
        got_o.append(o.cpu().numpy())
        got_l.append(l.cpu().numpy())
    got_o, got_l = np.stack(got_o), np.stack(got_l)
    for h in range(H):
        one = lambda x: x[0, h][None].astype(np.float64)
        o_ref, l_ref = oracle.path_attn_rows(one(inp["q"]), one(inp["k"]), one(inp["v"]), one(inp["w"]),
                                             one(inp["beta"]), None, scale, rows)
        _check(f"decode scale {scale} head {h}", dtype, got_o[:, 0, h], got_l[:, 0, h], o_ref, l_ref)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_partial_path(dtype, d):
    """Partial PaTH: the position transform acts on the first half of the
    head dimension only (w_t zero on the second half, unit norm on the first);
    the second half passes through unchanged (no position encoding)."""
    B, H, T = 1, 2, 256
    inp = workloads.small(dtype, B, H, T, d, seed=63, beta_sigma=1.5)
    w = inp["w"].astype(np.float64)
    w[..., d // 2:] = 0.0
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    inp["w"] = workloads.bf16_round(w.astype(np.float32)) if dtype == "bf16" else w.astype(np.float32)
    out, lse = run_hip(to_device(inp, dtype))
    o_ref, l_ref = oracle_full(inp)
    _check(f"partial PaTH {dtype} d={d}", dtype, out, lse, o_ref, l_ref)
