"""Pins of the fp64 gradient oracle (oracle/backward.py) against what does not
depend on it: the C oracle's forward pass (an independent walk), central
finite differences of that forward pass, and the textbook gradients of
softmax attention at beta = 0 (PaTH slides, frame "PaTH inserts a learned
transformation along every path": with beta = 0 every H_t is the identity)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import backward as ob


def _inputs(rng, T, d, fox):
    q, k, v = (rng.standard_normal((T, d)) for _ in range(3))
    w = rng.standard_normal((T, d))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    beta = rng.uniform(0.05, 1.95, size=T)
    logf = np.log(rng.uniform(0.5, 1.0, size=T)) if fox else None
    return dict(q=q, k=k, v=v, w=w, beta=beta, logf=logf)


def _loss_c(x, do, dlse):
    o, lse = oracle.path_attn(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"])
    return float(np.sum(o * do) + np.sum(lse * dlse))


@pytest.mark.parametrize("fox", [False, True])
def test_forward_equals_c_oracle(fox):
    import torch
    rng = np.random.default_rng(600 + fox)
    x = _inputs(rng, 21, 5, fox)
    t = lambda a: None if a is None else torch.tensor(a)
    o, lse = ob.forward(t(x["q"]), t(x["k"]), t(x["v"]), t(x["w"]), t(x["beta"]), t(x["logf"]))
    o_c, l_c = oracle.path_attn(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"])
    np.testing.assert_allclose(o.numpy(), o_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse.numpy(), l_c, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fox", [False, True])
def test_gradients_match_finite_differences(fox):
    rng = np.random.default_rng(610 + fox)
    T, d = 17, 4
    x = _inputs(rng, T, d, fox)
    do, dlse = rng.standard_normal((T, d)), rng.standard_normal(T)
    g = ob.gradients(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do, dlse)
    eps = 1e-6
    names = ["q", "k", "v", "w", "beta"] + (["logf"] if fox else [])
    for name in names:
        for _ in range(3):
            delta = rng.standard_normal(np.shape(x[name]))
            xp = dict(x); xp[name] = x[name] + eps * delta
            xm = dict(x); xm[name] = x[name] - eps * delta
            fd = (_loss_c(xp, do, dlse) - _loss_c(xm, do, dlse)) / (2 * eps)
            an = float(np.sum(g["d" + name] * delta))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_beta0_textbook_gradients():
    rng = np.random.default_rng(620)
    T, d = 19, 6
    x = _inputs(rng, T, d, False)
    x["beta"] = np.zeros(T)
    do, dlse = rng.standard_normal((T, d)), rng.standard_normal(T)
    g = ob.gradients(x["q"], x["k"], x["v"], x["w"], x["beta"], None, do, dlse)
    scale = 1.0 / np.sqrt(d)
    s = scale * x["q"] @ x["k"].T
    s[np.triu_indices(T, 1)] = -np.inf
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    o = p @ x["v"]
    dp = do @ x["v"].T
    ds = p * (dp - np.sum(do * o, 1, keepdims=True)) + p * dlse[:, None]
    np.testing.assert_allclose(g["dv"], p.T @ do, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dq"], scale * ds @ x["k"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk"], scale * ds.T @ x["q"], rtol=1e-10, atol=1e-12)
    assert np.all(g["dw"] == 0.0)


def test_first_token_factors_get_zero_gradient():
    """H_0 and f_0 enter no logit, so their gradients are exactly zero."""
    rng = np.random.default_rng(630)
    x = _inputs(rng, 9, 3, True)
    do = rng.standard_normal((9, 3))
    g = ob.gradients(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do)
    assert np.all(g["dw"][0] == 0.0) and g["dbeta"][0] == 0.0 and g["dlogf"][0] == 0.0


def test_pins_catch_reversed_product(monkeypatch):
    """A planted mistake in a copy of the oracle (the factors applied in the
    reverse order, H_i first for key j) must fail the finite-difference pin."""
    import torch

    def reversed_logits(q, k, w, beta):
        T = q.shape[0]
        c = torch.full((T, T), -torch.inf, dtype=q.dtype)
        out = []
        for i in range(T):
            row = []
            for j in range(T):
                if j > i:
                    row.append(torch.tensor(-torch.inf, dtype=q.dtype))
                    continue
                z = q[i]
                for t in range(j + 1, i + 1):      # H_{j+1} first: wrong order
                    z = z - beta[t] * (z @ w[t]) * w[t]
                row.append(z @ k[j])
            out.append(torch.stack(row))
        return torch.stack(out)

    monkeypatch.setattr(ob, "_logits", reversed_logits)
    with pytest.raises(AssertionError):
        test_gradients_match_finite_differences(False)


@pytest.mark.parametrize("C,n,d,fox", [(4, 4, 5, False), (4, 5, 3, True), (8, 3, 6, True), (1, 6, 3, False)])
def test_blockwise_backward_equals_autograd(C, n, d, fox):
    """The blockwise backward (oracle/chunked_backward.py: key levels, the
    downward sweep of the key-gradient accumulator, per-chunk adjoint of the
    UT formulas) gives the gradients of the definition."""
    from oracle import chunked_backward as cb
    rng = np.random.default_rng(640 + C + n)
    T = C * n
    x = _inputs(rng, T, d, fox)
    do, dlse = rng.standard_normal((T, d)), rng.standard_normal(T)
    ref = ob.gradients(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do, dlse)
    got = cb.sweep_backward(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do,
                            ref["o"], ref["lse"], dlse=dlse, C=C)
    for name in ("dq", "dk", "dv", "dw", "dbeta") + (("dlogf",) if fox else ()):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-9, atol=1e-10, err_msg=name)


@pytest.mark.parametrize("T,d,fox,near2", [(256, 64, False, 0.0), (384, 64, True, 0.0),
                                           (256, 128, True, 0.0), (320, 128, False, 0.1)])
def test_blockwise_backward_equals_autograd_at_chunk_64(T, d, fox, near2):
    """The same pin at the chunk length the GPU path and the full-size GPU
    tests use (C = 64), at the head dims 64 and 128 and 4-6 chunks, on inputs
    of the workloads' recipe (unit-norm w, beta = 2 sigmoid(N(0, 1.5)), 10 %
    of beta in [1.9, 2) in one case, log f = logsigmoid(N(3, 1)))."""
    import workloads
    from oracle import chunked_backward as cb
    x = workloads.small("f32", 1, 1, T, d, seed=650 + T + d, beta_sigma=1.5,
                        near2_frac=near2, fox=fox)
    x = {n: (None if a is None else np.asarray(a[0, 0], dtype=np.float64)) for n, a in x.items()}
    cot = workloads.cotangents("f32", 1, 1, T, d, seed=660 + T)
    do, dlse = cot["dout"][0, 0].astype(np.float64), cot["dlse"][0, 0].astype(np.float64)
    ref = ob.gradients(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do, dlse)
    got = cb.sweep_backward(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"], do,
                            ref["o"], ref["lse"], dlse=dlse, C=64)
    for name in ("dq", "dk", "dv", "dw", "dbeta") + (("dlogf",) if fox else ()):
        scale = max(1.0, float(np.max(np.abs(ref[name]))))
        np.testing.assert_allclose(got[name], ref[name], rtol=0, atol=1e-11 * scale, err_msg=name)
