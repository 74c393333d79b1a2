"""GPU parity of the PATH_ATTN_PRECISE option (bf16): the cross-chunk logits
take the running query tile as a bf16 hi + lo pair.

Sharp attention (q scaled by 3, logits three times larger) is where the
default's bf16 rounding of that tile shows: its lse error (about 1.6e-2, a
reported diagnostic in test_gpu_parity) exceeds the graded 1e-2.  With the
option it is held to the graded bars (o 2e-2, lse 1e-2) against the float64
oracle, at d = 64 and 128, with and without the gate.  The option keeps the
forget-gate skip exact (bitwise equal to every block computed) and changes
nothing for float32 inputs (bitwise equal to the default).
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import TOL, oracle_full, record, to_device

pytestmark = pytest.mark.gpu


def _fwd(dev, flags):
    import torch
    import householder_position_encoding_amd as pa
    out, lse = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"],
                                flags=flags)
    torch.cuda.synchronize()
    return out, lse


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,fox,T", [(64, False, 256), (64, True, 1024), (128, False, 256),
                                     (128, True, 640)])
def test_precise_sharp_attention_meets_graded_bars(d, fox, T):
    import householder_position_encoding_amd as pa
    inp = workloads.small("bf16", 1, 2, T, d, seed=7 + T + d, q_scale=3.0, fox=fox)
    dev = to_device(inp, "bf16")
    o_ref, l_ref = oracle_full(inp)
    out_p, lse_p = _fwd(dev, pa.PRECISE)
    out_d, lse_d = _fwd(dev, 0)
    ep_o, ep_l = float(np.max(np.abs(_np(out_p) - o_ref))), float(np.max(np.abs(_np(lse_p) - l_ref)))
    ed_o, ed_l = float(np.max(np.abs(_np(out_d) - o_ref))), float(np.max(np.abs(_np(lse_d) - l_ref)))
    record(f"precise sharp q x3 d{d} fox={fox} T={T}", max_abs_err_o=ep_o, max_abs_err_lse=ep_l,
           default_max_abs_err_o=ed_o, default_max_abs_err_lse=ed_l)
    print(f"sharp d{d} fox={fox} T={T}: precise o {ep_o:.3g} lse {ep_l:.3g}; default o {ed_o:.3g} lse {ed_l:.3g}")
    tol_o, tol_l = TOL["bf16"]
    assert ep_o <= tol_o and ep_l <= tol_l


@pytest.mark.parametrize("d", [64, 128])
def test_precise_skip_is_exact(d):
    """With the gate the precise kernel skips blocks whose weights are all
    exactly zero: the outputs equal those with every block computed."""
    import torch
    import householder_position_encoding_amd as pa
    inp = workloads.small("bf16", 1, 2, 2048, d, seed=99 + d, fox=True)
    dev = to_device(inp, "bf16")
    out_s, lse_s = _fwd(dev, pa.PRECISE)
    out_n, lse_n = _fwd(dev, pa.PRECISE | pa.NO_SKIP)
    assert torch.equal(lse_s, lse_n)
    assert torch.equal(out_s.float(), out_n.float())   # -0 and +0 compare equal


def test_precise_leaves_float32_unchanged():
    import torch
    import householder_position_encoding_amd as pa
    inp = workloads.small("f32", 1, 2, 256, 64, seed=5, fox=True)
    dev = to_device(inp, "f32")
    out_p, lse_p = _fwd(dev, pa.PRECISE)
    out_d, lse_d = _fwd(dev, 0)
    assert torch.equal(out_p, out_d) and torch.equal(lse_p, lse_d)
