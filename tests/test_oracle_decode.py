"""Pins of the decoding oracle (oracle/decode.py) against what the pages and
mathematics fix, and planted mistakes that those pins must catch.

PaTH slides, frame "Decoding updates historical keys in place" (Sec. 3.4,
Eq. 1): refined keys dotted with the current query are the path logits, which
the C oracle computes by an independent walk over the query (and which
tests/test_oracle_pins.py pins to closed forms and brute force).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import decode


def _inputs(rng, T, d, unit=True):
    q, k = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    w = rng.standard_normal((T, d))
    if unit:
        w /= np.linalg.norm(w, axis=1, keepdims=True)
    beta = rng.uniform(0.0, 2.0, size=T)
    return q, k, w, beta


def pin_refined_keys_give_path_logits(refined):
    rng = np.random.default_rng(400)
    T, d = 37, 6
    q, k, w, beta = _inputs(rng, T, d)
    S = oracle.path_logits(q, k, w, beta)
    for upto in (0, 1, 17, T - 1):
        kr = refined(k, w, beta, upto)
        assert kr.shape == (upto + 1, d)
        np.testing.assert_allclose(kr @ q[upto], S[upto, :upto + 1], rtol=1e-12, atol=1e-12)


def pin_beta0_identity(refined):
    rng = np.random.default_rng(401)
    q, k, w, _ = _inputs(rng, 12, 5)
    kr = refined(k, w, np.zeros(12), 11)
    assert np.array_equal(kr, k)


def pin_reflections_preserve_norm(refined):
    rng = np.random.default_rng(402)
    q, k, w, _ = _inputs(rng, 15, 4)
    kr = refined(k, w, np.full(15, 2.0), 14)
    np.testing.assert_allclose(np.linalg.norm(kr, axis=1), np.linalg.norm(k, axis=1), rtol=1e-12)


def pin_single_step(refined):
    """Two tokens: key 0 aligned to position 1 is H_1 k_0, written out."""
    k = np.array([[1.0, 2.0, -1.0], [0.5, 0.0, 3.0]])
    w = np.array([[0.0, 0.0, 1.0], [0.6, 0.8, 0.0]])
    beta = np.array([0.3, 1.5])
    kr = refined(k, w, beta, 1)
    # w_1 . k_0 = 0.6 + 1.6 = 2.2; H_1 k_0 = k_0 - 1.5 * 2.2 * w_1
    np.testing.assert_allclose(kr[0], [1.0 - 1.98, 2.0 - 2.64, -1.0], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(kr[1], k[1])


REFINED_PINS = [pin_refined_keys_give_path_logits, pin_beta0_identity,
                pin_reflections_preserve_norm, pin_single_step]


@pytest.mark.parametrize("pin", REFINED_PINS, ids=lambda f: f.__name__[4:])
def test_refined_keys_pin(pin):
    pin(decode.refined_keys)


def _aligned_rows_all(k, w, beta, upto):
    return decode.aligned_key_rows(k, w, beta, range(upto + 1), upto)


@pytest.mark.parametrize("pin", REFINED_PINS, ids=lambda f: f.__name__[4:])
def test_aligned_key_rows_pin(pin):
    """The per-row alignment (used to sample full-length caches) meets the
    same pins as the whole-cache recurrence."""
    pin(_aligned_rows_all)


def test_aligned_key_rows_sample_subset():
    rng = np.random.default_rng(404)
    q, k, w, beta = _inputs(rng, 40, 7)
    rows = [0, 3, 39, 17]
    np.testing.assert_allclose(decode.aligned_key_rows(k, w, beta, rows, 39),
                               decode.refined_keys(k, w, beta, 39)[rows], rtol=1e-12, atol=1e-12)


def test_gate_prefix():
    rng = np.random.default_rng(403)
    logf = -rng.uniform(0.0, 1.0, size=(2, 3, 9))
    lam = decode.gate_prefix(logf)
    assert np.all(lam[..., 0] == 0.0)
    for t in range(9):
        for j in range(t + 1):
            np.testing.assert_allclose(lam[..., t] - lam[..., j],
                                       logf[..., j + 1:t + 1].sum(-1), rtol=1e-12, atol=1e-12)


# ---- planted mistakes (in copies of the oracle, on the CPU): each must fail a pin

def _wrong_order(k, w, beta, upto):
    """Applies the reflections newest-first (H_{j+1} last instead of first)."""
    k = np.array(k[: upto + 1], dtype=np.float64)
    for j in range(upto + 1):
        z = k[j].copy()
        for t in range(upto, j, -1):
            z -= beta[t] * (w[t] @ z) * w[t]
        k[j] = z
    return k


def _includes_own_reflection(k, w, beta, upto):
    """Also reflects key t by its own H_t."""
    k = np.array(k[: upto + 1], dtype=np.float64)
    for t in range(1, upto + 1):
        k[: t + 1] -= beta[t] * np.outer(k[: t + 1] @ w[t], w[t])
    return k


def _sign_flip(k, w, beta, upto):
    k = np.array(k[: upto + 1], dtype=np.float64)
    for t in range(1, upto + 1):
        k[:t] += beta[t] * np.outer(k[:t] @ w[t], w[t])
    return k


def _half_beta(k, w, beta, upto):
    return decode.refined_keys(k, w, 0.5 * np.asarray(beta), upto)


@pytest.mark.parametrize("mutant", [_wrong_order, _includes_own_reflection, _sign_flip, _half_beta],
                         ids=lambda f: f.__name__[1:])
def test_refined_key_pins_catch_mutant(mutant):
    failed = False
    for pin in REFINED_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed = True
    assert failed, f"no pin caught {mutant.__name__}"
