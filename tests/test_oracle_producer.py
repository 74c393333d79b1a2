"""Pins of the fp64 w / beta producer oracle (oracle/producer.py).

Each check rests on something other than the oracle's own formulas: the
hand-worked example in tests/golden/producer_tiny.txt, the unit norm the
pages require of w_t, the reach of a causal width-3 convolution, the scale
and sign behaviour of a normalisation, the shift a one-tap convolution makes,
and closed forms of 2 sigmoid.
"""
from __future__ import annotations

import math
import os

import numpy as np

from oracle.producer import producer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "producer_tiny.txt")


def _case(seed, B=2, T=11, Dm=12, R=5, H=3, d=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, Dm))
    Wd = rng.standard_normal((R, Dm)) / math.sqrt(Dm)
    Wu = rng.standard_normal((H * d, R)) / math.sqrt(R)
    cw = rng.standard_normal((H * d, 3))
    u = rng.standard_normal((H, Dm)) / math.sqrt(Dm)
    ub = rng.standard_normal(H)
    return x, Wd, Wu, cw, u, ub, H, d


def test_hand_worked_example():
    rows = np.loadtxt(GOLDEN)
    x = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])
    Wd = np.array([[1.0, 2.0]])
    Wu = np.array([[3.0], [4.0]])
    cw = np.array([[1.0, 1.0, 1.0], [0.0, 0.0, 1.0]])
    u = np.array([[1.0, -1.0]])
    ub = np.array([0.0])
    w, beta = producer(x, Wd, Wu, cw, u, ub, H=1, d=2)
    np.testing.assert_allclose(w[0, 0], rows[:, 1:3], rtol=0, atol=1e-15)
    np.testing.assert_allclose(beta[0, 0], rows[:, 3], rtol=0, atol=1e-15)


def test_unit_norm_per_head():
    """||w_t||_2 = 1 for every head separately (heads of different sizes
    before the normalisation, so a normalisation over all heads fails)."""
    x, Wd, Wu, cw, u, ub, H, d = _case(1)
    Wu[:d] *= 10.0
    w, _ = producer(x, Wd, Wu, cw, u, ub, H, d)
    np.testing.assert_allclose(np.linalg.norm(w, axis=-1), 1.0, rtol=0, atol=1e-13)


def test_zero_vector_gives_zero_w():
    x, Wd, Wu, cw, u, ub, H, d = _case(2)
    x[:, 0] = 0.0   # z_0 = 0, so z'_0 = 0 (no earlier tokens)
    w, _ = producer(x, Wd, Wu, cw, u, ub, H, d)
    assert np.all(w[:, :, 0] == 0.0)


def test_convolution_reaches_two_tokens_ahead_only():
    """Brute force: changing x_s changes w_t only for t in {s, s+1, s+2} and
    beta only at s (causal, width 3)."""
    x, Wd, Wu, cw, u, ub, H, d = _case(3)
    w0, b0 = producer(x, Wd, Wu, cw, u, ub, H, d)
    s = 4
    x2 = x.copy()
    x2[:, s] += 0.5
    w1, b1 = producer(x2, Wd, Wu, cw, u, ub, H, d)
    changed_w = np.any(np.abs(w1 - w0) > 1e-12, axis=(0, 1, 3))
    changed_b = np.any(np.abs(b1 - b0) > 1e-12, axis=(0, 1))
    assert changed_w.tolist() == [t in (s, s + 1, s + 2) for t in range(x.shape[1])]
    assert changed_b.tolist() == [t == s for t in range(x.shape[1])]


def test_normalisation_scale_and_sign():
    """w is invariant to a positive scale of the projection and flips with
    its sign."""
    x, Wd, Wu, cw, u, ub, H, d = _case(4)
    w0, _ = producer(x, Wd, Wu, cw, u, ub, H, d)
    w1, _ = producer(x, Wd, 7.5 * Wu, cw, u, ub, H, d)
    w2, _ = producer(x, Wd, -Wu, cw, u, ub, H, d)
    np.testing.assert_allclose(w1, w0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(w2, -w0, rtol=0, atol=1e-13)


def test_one_tap_convolution_is_a_shift():
    """Taps (1, 0, 0) read the token two back: their w at t is the w of taps
    (0, 0, 1) at t - 2, and zero at t < 2."""
    x, Wd, Wu, cw, u, ub, H, d = _case(5)
    old = np.zeros_like(cw)
    old[:, 0] = 1.0
    cur = np.zeros_like(cw)
    cur[:, 2] = 1.0
    wo, _ = producer(x, Wd, Wu, old, u, ub, H, d)
    wc, _ = producer(x, Wd, Wu, cur, u, ub, H, d)
    np.testing.assert_allclose(wo[:, :, 2:], wc[:, :, :-2], rtol=0, atol=1e-15)
    assert np.all(wo[:, :, :2] == 0.0)


def test_beta_closed_forms():
    """2 sigmoid(0) = 1 and 2 sigmoid(ln 3) = 3/2, exactly; beta in (0, 2)."""
    x, Wd, Wu, cw, u, ub, H, d = _case(6)
    _, b = producer(x, Wd, Wu, cw, np.zeros_like(u), np.zeros(H), H, d)
    assert np.all(b == 1.0)
    _, b = producer(x, Wd, Wu, cw, np.zeros_like(u), np.full(H, math.log(3.0)), H, d)
    np.testing.assert_allclose(b, 1.5, rtol=0, atol=1e-15)
    _, b = producer(x, Wd, Wu, cw, u, ub, H, d)
    assert np.all((b > 0.0) & (b < 2.0))
