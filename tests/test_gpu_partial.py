"""Partial PaTH on the GPU (path_attn_fwd_partial) against the fp64 oracle.

The authors' response page remarks that PaTH can be applied to part of the
head dimensions for speed.  With d_path = d / 2 the factors act on the leading
d_path coordinates: H_t = I - beta_t w~ w~^T with w~ = (w_t[:d_path], 0).
The GPU gets w with random trailing coordinates (which it must not read);
the oracle gets the same w with them set to zero, i.e. the definition of the
PaTH slides (frame "PaTH inserts a learned transformation along every path")
applied to w~.  Bars as for the forward: 1e-4 (float32), 2e-2 on o and 1e-2
on lse (bf16); every row for the small cases, sampled rows of nine heads for
the full-size one.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import (TOL, oracle_full, oracle_rows, record, sample_rows, spread_heads,
                            to_device)

pytestmark = pytest.mark.gpu


def _zero_tail(inp, d_path):
    ref = dict(inp)
    w = inp["w"].copy()
    w[..., d_path:] = 0.0
    ref["w"] = w
    return ref


def _run(dev, d_path):
    import torch
    import householder_position_encoding_amd as pa
    out, lse = pa.path_attn_fwd_partial(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"],
                                        dev["logf"], d_path=d_path)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(name, dtype, out, lse, o_ref, l_ref):
    tol_o, tol_l = TOL[dtype]
    eo = float(np.max(np.abs(out - o_ref)))
    el = float(np.max(np.abs(lse - l_ref)))
    record(name, max_abs_err_o=eo, max_abs_err_lse=el, rows=int(np.prod(np.shape(lse))))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= tol_o and el <= tol_l, (name, eo, el)


CASES = [
    ("bf16", 64, False, 1, 2, 576, {"beta_sigma": 1.5}),
    ("bf16", 64, True, 2, 2, 512, {}),
    ("bf16", 64, False, 1, 2, 200, {}),                       # ragged
    ("bf16", 128, False, 1, 2, 384, {"beta_sigma": 1.5, "near2_frac": 0.1}),
    ("bf16", 128, True, 1, 2, 640, {}),
    ("f32", 64, False, 1, 2, 320, {}),
    ("f32", 128, True, 1, 2, 256, {}),
    ("f32", 64, False, 1, 1, 256, {"beta_const": 2.0}),       # exact reflections on half the dims
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-d{c[1]}-fox{int(c[2])}-t{c[5]}")
def test_partial_path_all_rows(case):
    dtype, d, fox, B, H, T, opts = case
    d_path = d // 2
    inp = workloads.small(dtype, B, H, T, d, seed=401 + T + d, fox=fox, **opts)
    out, lse = _run(to_device(inp, dtype), d_path)
    o_ref, l_ref = oracle_full(_zero_tail(inp, d_path))
    _check(f"partial d_path={d_path} {case}", dtype, out, lse, o_ref, l_ref)


def test_partial_path_full_dims_equals_path_attn_fwd():
    """d_path = d runs the ordinary forward: the same bits as path_attn_fwd."""
    import torch
    import householder_position_encoding_amd as pa
    inp = workloads.small("bf16", 1, 2, 320, 64, seed=411, fox=True)
    dev = to_device(inp, "bf16")
    o1, l1 = pa.path_attn_fwd_partial(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"],
                                      dev["logf"], d_path=64)
    o2, l2 = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_partial_path_benchmark_shape():
    """The benchmark workload's shape (bf16 B2 H16 T16384 d64) with d_path = 32:
    sampled rows of nine heads against the oracle."""
    wl = workloads.LONG_D64
    inp = workloads.generate(wl)
    out, lse = _run(to_device(inp, "bf16"), 32)
    ref = _zero_tail(inp, 32)
    rng = np.random.default_rng(77)
    heads = spread_heads(wl.B, wl.H)
    rows = [sample_rows(wl.T, rng, n_random=48) for _ in heads]
    o_ref, l_ref = oracle_rows(ref, heads, rows)
    got_o = np.concatenate([out[b, h, r] for (b, h), r in zip(heads, rows)])
    got_l = np.concatenate([lse[b, h, r] for (b, h), r in zip(heads, rows)])
    _check("partial d_path=32 bf16_b2h16t16384d64", "bf16", got_o, got_l, o_ref, l_ref)
