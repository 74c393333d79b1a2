"""GPU parity of the w / beta producer (path_attn_wbeta) against the fp64
oracle (oracle/producer.py), element by element.

Inputs are bf16 (x and the three projections, exact in bf16) with float32
taps and bias; the oracle takes the same rounded values in float64.

Bar: |w - w_ref| <= 3e-3 per element (w has unit rows: its bf16 rounding is
at most 2^-9 ~ 2.0e-3 of an element's size; the products before it keep
float32 accumulation and the low-rank intermediate as a hi/lo pair, about 1e-6
relative) and |beta - beta_ref| <= 5e-5 (float32 sums of Dm products and the
exponential, about 1e-6).  Rows whose vector is zero must give w = 0 exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle.producer import producer
from tests.gpu_util import record

pytestmark = pytest.mark.gpu

TOL_W, TOL_BETA = 3e-3, 5e-5


def _bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _inputs(B, T, Dm, R, H, d, seed):
    """Seeded bf16 inputs (x ~ N(0, 1); projections scaled by 1/sqrt(fan-in);
    taps ~ N(0, 1/3); beta's bias ~ N(0, 1)) and their float64 values."""
    import torch
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((B, T, Dm)))
    wd = _bf16(rng.standard_normal((R, Dm)) / math.sqrt(Dm))
    wu = _bf16(rng.standard_normal((H * d, R)) / math.sqrt(R))
    u = _bf16(rng.standard_normal((H, Dm)) / math.sqrt(Dm))
    cw = torch.from_numpy((rng.standard_normal((H * d, 3)) / math.sqrt(3)).astype(np.float32))
    ub = torch.from_numpy(rng.standard_normal(H).astype(np.float32))
    f64 = lambda t: t.float().numpy().astype(np.float64)
    host = dict(x=x, wd=wd, wu=wu, cw=cw, u=u, ub=ub)
    ref = {k: f64(v) for k, v in host.items()}
    return host, ref


def _run(host, H, d):
    import torch
    import householder_position_encoding_amd as pa
    dev = {k: v.cuda().contiguous() for k, v in host.items()}
    w, beta = pa.path_attn_wbeta(dev["x"], dev["wd"], dev["wu"], dev["cw"], dev["u"], dev["ub"], H, d)
    torch.cuda.synchronize()
    return w.float().cpu().numpy().astype(np.float64), beta.cpu().numpy().astype(np.float64)


CASES = [
    # B, T, Dm, R, H, d
    (2, 130, 64, 32, 2, 64),     # three tiles, ragged
    (1, 62, 192, 48, 2, 64),     # exactly one tile
    (1, 1, 64, 16, 1, 64),       # a single token
    (1, 200, 128, 64, 3, 128),
    (2, 125, 64, 128, 1, 128),   # R at its maximum
    (2, 190, 128, 96, 2, 64),    # d = 64 with R past 64 (the wider Wu staging)
    (1, 100, 192, 32, 3, 64),    # an odd head count: the last head alone; Dm of three chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_producer_matches_oracle(case):
    B, T, Dm, R, H, d = case
    host, ref = _inputs(B, T, Dm, R, H, d, seed=300 + T + d)
    w, beta = _run(host, H, d)
    w_ref, b_ref = producer(ref["x"], ref["wd"], ref["wu"], ref["cw"], ref["u"], ref["ub"], H, d)
    ew, eb = float(np.max(np.abs(w - w_ref))), float(np.max(np.abs(beta - b_ref)))
    record(f"producer {case}", max_abs_err_w=ew, max_abs_err_beta=eb, tol_w=TOL_W, tol_beta=TOL_BETA)
    assert ew <= TOL_W and eb <= TOL_BETA
    # unit rows
    np.testing.assert_allclose(np.linalg.norm(w, axis=-1), 1.0, rtol=0, atol=5e-3)


def test_producer_zero_rows_give_zero_w():
    """Tokens 0..69 all zero: z' is zero for tokens 0..69 (the taps reach two
    tokens back, all zero), so w must be exactly zero there, across the first
    tile boundary; beta there is 2 sigmoid(ub) (x = 0)."""
    import torch
    B, T, Dm, R, H, d = 1, 150, 64, 32, 2, 64
    host, ref = _inputs(B, T, Dm, R, H, d, seed=77)
    host["x"][:, :70] = 0
    ref["x"][:, :70] = 0.0
    w, beta = _run(host, H, d)
    assert np.all(w[:, :, :70] == 0.0)
    w_ref, b_ref = producer(ref["x"], ref["wd"], ref["wu"], ref["cw"], ref["u"], ref["ub"], H, d)
    assert float(np.max(np.abs(w - w_ref))) <= TOL_W
    assert float(np.max(np.abs(beta - b_ref))) <= TOL_BETA
    np.testing.assert_allclose(beta[0, :, 0], 2.0 / (1.0 + np.exp(-ref["ub"])), rtol=0, atol=TOL_BETA)


def test_producer_full_size_sampled_tokens():
    """The benchmark shape: B2 T16384, H16 d64 from hidden size Dm = H d = 1024,
    rank R = 64; every head of 321 tokens of each batch row: those around
    every seventh tile boundary (a block covers 62 tokens), 212 at random and
    the last."""
    B, T, Dm, R, H, d = 2, 16384, 1024, 64, 16, 64
    host, ref = _inputs(B, T, Dm, R, H, d, seed=2024)
    w, beta = _run(host, H, d)
    rng = np.random.default_rng(5)
    bounds = [t for k in range(0, T // 62 + 1, 7) for t in (62 * k - 1, 62 * k, 62 * k + 1) if 0 <= t < T]
    toks = np.array(sorted(set(bounds[:300]) | set(rng.choice(T, 212, replace=False).tolist()) | {T - 1}))
    # the oracle on the window of tokens each sample needs (itself and two before)
    ew = eb = 0.0
    for t in toks:
        lo = max(0, t - 2)
        xs = ref["x"][:, lo:t + 1]
        w_ref, b_ref = producer(xs, ref["wd"], ref["wu"], ref["cw"], ref["u"], ref["ub"], H, d)
        ew = max(ew, float(np.max(np.abs(w[:, :, t] - w_ref[:, :, -1]))))
        eb = max(eb, float(np.max(np.abs(beta[:, :, t] - b_ref[:, :, -1]))))
    record("producer B2 T16384 Dm1024 R64 H16 d64 (sampled tokens)", max_abs_err_w=ew,
           max_abs_err_beta=eb, tokens=int(len(toks)), tol_w=TOL_W, tol_beta=TOL_BETA)
    assert ew <= TOL_W and eb <= TOL_BETA
