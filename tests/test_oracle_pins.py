"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each ``pin_*`` function takes the loaded oracle library so that
``test_oracle_mutants.py`` can run the same pins against copies of the oracle
with a planted mistake and show that some pin fails for each.

Sources (PaTH discussion slides, arXiv:2505.16381v2; author-response page):
  * frame "PaTH inserts a learned transformation along every path" (Sec. 2.2):
    the logit definition and the softmax / value sum;
  * frame "One direction can shrink, disappear, or change sign": action of H_t;
  * frame "PaTH keeps a recurrent path and a softmax readout": linear RNN;
  * frame "A reflection can implement a symbolic swap": beta = 2 swap;
  * frame "FoX adds a separate mechanism for forgetting": the gate;
  * frame "A triangular representation makes paths computable": UT form;
  * frame "Decoding updates historical keys in place" (Sec. 3.4, Eq. 1);
  * author-response page, "Implementation detail": scale and -inf mask.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
from scipy.linalg import solve_triangular

import oracle
from oracle.chunked import chunk_quantities, chunked_logits, ut_chunk_quantities

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, T, d, beta_lo=0.0, beta_hi=2.0):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    w = rng.standard_normal((T, d))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    beta = rng.uniform(beta_lo, beta_hi, size=T)
    return q, k, v, w, beta


def _textbook_attention(S, v):
    """Row softmax of a masked logit matrix and the value sum (fp64)."""
    m = np.max(S, axis=1, keepdims=True)
    P = np.exp(S - m)
    Z = P.sum(axis=1, keepdims=True)
    return (P / Z) @ v, (m + np.log(Z))[:, 0]


def _causal(S):
    T = S.shape[0]
    return np.where(np.tril(np.ones((T, T), dtype=bool)), S, -np.inf)


def _dense_H(w_t, beta_t):
    d = w_t.shape[0]
    return np.eye(d) - beta_t * np.outer(w_t, w_t)


# ---------------------------------------------------------------- pins

def pin_beta0_is_causal_attention(lib):
    """beta = 0 makes every H_t the identity: ordinary causal softmax
    attention with scale 1/sqrt(d)."""
    rng = np.random.default_rng(100)
    T, d = 40, 8
    q, k, v, w, _ = _rand_inputs(rng, T, d)
    beta = np.zeros(T)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle.path_attn(q, k, v, w, beta, scale=scale, lib=lib)
    o_ref, lse_ref = _textbook_attention(_causal(scale * q @ k.T), v)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def pin_beta0_fox_is_forgetting_attention(lib):
    """beta = 0 with a forget gate: logit scale q_i.k_j + sum_{s=j+1..i} log f_s,
    the gate outside the scale (FoX frame)."""
    rng = np.random.default_rng(101)
    T, d = 37, 8
    q, k, v, w, _ = _rand_inputs(rng, T, d)
    beta = np.zeros(T)
    logf = -rng.uniform(0.0, 0.7, size=T)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle.path_attn(q, k, v, w, beta, logf, scale=scale, lib=lib)
    Lam = np.cumsum(logf)
    gate = Lam[:, None] - Lam[None, :]
    o_ref, lse_ref = _textbook_attention(_causal(scale * q @ k.T + gate), v)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def pin_swap_closed_form(lib):
    """beta = 2 and w_t = (e_a - e_b)/sqrt(2): H_t swaps coordinates a and b,
    so c_ij = k_j . (q_i with the swaps of t = i, i-1, ..., j+1 applied)."""
    rng = np.random.default_rng(102)
    T, d = 24, 6
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    pairs = []
    w = np.zeros((T, d))
    for t in range(T):
        a, b = rng.choice(d, size=2, replace=False)
        pairs.append((a, b))
        w[t, a], w[t, b] = 1.0 / np.sqrt(2.0), -1.0 / np.sqrt(2.0)
    beta = np.full(T, 2.0)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    for i in range(T):
        z = q[i].copy()
        for j in range(i, -1, -1):
            assert abs(S[i, j] - k[j] @ z) <= 1e-12 * (1 + abs(k[j] @ z))
            if j == 0:
                break
            a, b = pairs[j]
            z[a], z[b] = z[b], z[a]


def pin_swap_golden(lib):
    """The hand-worked five-coordinate swap chain stored in tests/golden."""
    swaps, logits = [], []
    with open(os.path.join(GOLDEN, "swap_chain_d5.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] == "swap":
                swaps.append((int(p[1]), int(p[2]) - 1, int(p[3]) - 1))
            elif p[0] == "logit":
                logits.append((int(p[1]), int(p[2]), float(p[3])))
    T, d = 4, 5
    w = np.zeros((T, d))
    w[0, 0] = 1.0  # H_0 never enters a logit; any unit vector
    for t, a, b in swaps:
        w[t, a], w[t, b] = 1.0 / np.sqrt(2.0), -1.0 / np.sqrt(2.0)
    beta = np.full(T, 2.0)
    q = np.zeros((T, d))
    q[3] = [1, 2, 3, 4, 5]
    k = np.tile([1.0, 10.0, 100.0, 1000.0, 10000.0], (T, 1))
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    for i, j, val in logits:
        assert abs(S[i, j] - val) <= 1e-9, (i, j, S[i, j], val)


def pin_dense_products(lib):
    """Explicit d x d matrices: c_ij = k_j^T (H_{j+1} H_{j+2} ... H_i) q_i."""
    rng = np.random.default_rng(103)
    T, d = 16, 5
    q, k, _, w, beta = _rand_inputs(rng, T, d)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    for i in range(T):
        for j in range(i + 1):
            P = np.eye(d)
            for t in range(j + 1, i + 1):      # left to right: H_{j+1} ... H_i
                P = P @ _dense_H(w[t], beta[t])
            ref = k[j] @ P @ q[i]
            assert abs(S[i, j] - ref) <= 1e-12 * (1 + abs(ref)), (i, j)
        assert np.all(np.isneginf(S[i, i + 1:]))


def pin_linear_rnn(lib):
    """S_t = S_{t-1} H_t + v_t k_t^T, o_t = S_t q_t unrolls to
    sum_j v_j c_tj; with one-hot v_t = e_t the entries of S_t q_t are c_tj."""
    rng = np.random.default_rng(104)
    T, d = 20, 6
    q, k, _, w, beta = _rand_inputs(rng, T, d)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    state = np.zeros((T, d))
    for t in range(T):
        state = state @ _dense_H(w[t], beta[t])
        state[t] += k[t]
        c = state @ q[t]
        np.testing.assert_allclose(S[t, :t + 1], c[:t + 1], rtol=1e-12, atol=1e-12)


def pin_decode_key_refinement(lib):
    """Decoding: k_j <- k_j - beta_t w_t (w_t . k_j) for j < t, append k_t,
    then (k_j^(t))^T q_t = c_tj (Sec. 3.4, Eq. 1)."""
    rng = np.random.default_rng(105)
    T, d = 20, 7
    q, k, _, w, beta = _rand_inputs(rng, T, d)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    cache = np.zeros((0, d))
    for t in range(T):
        if t > 0:
            cache = cache - beta[t] * np.outer(cache @ w[t], w[t])
        cache = np.vstack([cache, k[t]])
        np.testing.assert_allclose(S[t, :t + 1], cache @ q[t], rtol=1e-12, atol=1e-12)


def pin_global_ut_formula(lib):
    """A~ = lower(Q K^T) - lower(Q W^T) U strictLower(W K^T) with
    U = (I + strictLower(D W W^T))^{-1} D from a library triangular solve."""
    rng = np.random.default_rng(106)
    T, d = 30, 8
    q, k, _, w, beta = _rand_inputs(rng, T, d)
    D = np.diag(beta)
    U = solve_triangular(np.eye(T) + np.tril(D @ w @ w.T, -1), D, lower=True)
    A = np.tril(q @ k.T) - np.tril(q @ w.T) @ U @ np.tril(w @ k.T, -1)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    low = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(S[low], A[low], rtol=1e-11, atol=1e-11)


def pin_chunked_algorithm(lib):
    """The blockwise right-to-left scan reproduces the definition for several
    chunk sizes (C = 1 is the walk itself), including the chunk length 64 of
    the GPU path."""
    rng = np.random.default_rng(107)
    for T, d, Cs in ((32, 6, (1, 2, 4, 16)), (192, 8, (64,))):
        q, k, _, w, beta = _rand_inputs(rng, T, d)
        S = oracle.path_logits(q, k, w, beta, lib=lib)
        low = np.tril(np.ones((T, T), dtype=bool))
        for C in Cs:
            A = chunked_logits(q, k, w, beta, C)
            np.testing.assert_allclose(S[low], A[low], rtol=1e-11, atol=1e-11)
            assert np.all(A[~low] == -np.inf)


def pin_chunk_quantities(lib):
    """Per-chunk quantities: the definitions (explicit products of the H_t)
    agree with the UT form of the backup frame (U from a library triangular
    solve), and the diagonal-block logits and the moved queries and keys agree
    with the walk: Al[i, j] is the path logit c_ij of the chunk alone, <-Q row
    i is the walk of q_i down to the chunk start, and ->K row j dotted with a
    query moved to the chunk end gives the path logit from that end."""
    rng = np.random.default_rng(110)
    C, d = 24, 7
    q, k, _, w, beta = _rand_inputs(rng, C, d)
    got = chunk_quantities(q, k, w, beta)
    ut = ut_chunk_quantities(q, k, w, beta)
    low = np.tril(np.ones((C, C), dtype=bool))
    for name in ("qa", "kb", "m"):
        np.testing.assert_allclose(got[name], ut[name], rtol=1e-12, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(got["al"][low], ut["al"][low], rtol=1e-12, atol=1e-12)
    S = oracle.path_logits(q, k, w, beta, lib=lib)
    np.testing.assert_allclose(got["al"][low], S[low], rtol=1e-12, atol=1e-12)
    # with one token put before the chunk, the walk of row i + 1 down to that
    # token has crossed H_first ... H_i of the chunk: <-Q row i
    q1, w1 = np.vstack([np.zeros((1, d)), q]), np.vstack([w[:1], w])
    for i in (0, 5, C - 1):
        Z = oracle.path_walk(q1, w1, np.append(0.0, beta), i + 1, lib=lib)
        np.testing.assert_allclose(got["qa"][i], Z[i + 1], rtol=1e-12, atol=1e-12)
    # a query placed just after the chunk (beta = 0 for it) sees key j through
    # H_{j+1} ... H_last, i.e. through ->K row j
    q2 = np.vstack([q, rng.standard_normal((1, d))])
    k2 = np.vstack([k, np.zeros((1, d))])
    w2 = np.vstack([w, w[:1]])
    S2 = oracle.path_logits(q2, k2, w2, np.append(beta, 0.0), lib=lib)
    np.testing.assert_allclose(S2[C, :C], got["kb"] @ q2[C], rtol=1e-12, atol=1e-12)
    # the backup frame's transposed UT factor gives F itself
    np.testing.assert_allclose(got["F"], np.eye(d) - w.T @ ut["U"].T @ w, rtol=1e-12, atol=1e-12)


def pin_softmax_readout(lib):
    """o_i and lse_i are the row softmax of scale * c_ij + gate and the value
    sum, for a general beta (textbook softmax over the oracle's own logits)."""
    rng = np.random.default_rng(108)
    T, d = 33, 8
    q, k, v, w, beta = _rand_inputs(rng, T, d)
    logf = -rng.uniform(0.0, 0.5, size=T)
    scale = 1.0 / np.sqrt(d)
    S = oracle.path_logits(q, k, w, beta, logf, scale=scale, lib=lib)
    raw = oracle.path_logits(q, k, w, beta, lib=lib)
    Lam = np.cumsum(logf)
    low = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(S[low], (scale * raw + Lam[:, None] - Lam[None, :])[low],
                               rtol=1e-12, atol=1e-12)
    o, lse = oracle.path_attn(q, k, v, w, beta, logf, scale=scale, lib=lib)
    o_ref, lse_ref = _textbook_attention(S, v)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def pin_eigen_direction_golden(lib):
    """H_t z = z_perp + (1 - beta_t) alpha w_t, from tests/golden."""
    rows = np.loadtxt(os.path.join(GOLDEN, "eigen_direction_d3.txt"))
    for beta_t, *hz in rows:
        q = np.array([[0.0, 0.0, 0.0], [2.0, 3.0, 4.0]])
        w = np.array([[1.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
        Z = oracle.path_walk(q, w, np.array([0.0, beta_t]), 1, lib=lib)
        np.testing.assert_allclose(Z[0], q[1], rtol=0, atol=0)
        np.testing.assert_allclose(Z[1], hz, rtol=0, atol=1e-15)


def pin_walk_invariants(lib):
    """With unit w and beta in [0, 2] the spectral norm of H_t is <= 1, so
    ||z|| never grows along the walk; beta = 2 preserves it exactly; beta = 1
    erases the w_t component (author-response page; eigen frame)."""
    rng = np.random.default_rng(109)
    T, d = 50, 16
    q, _, _, w, beta = _rand_inputs(rng, T, d)
    Z = oracle.path_walk(q, w, beta, T - 1, lib=lib)
    n = np.linalg.norm(Z, axis=1)
    assert np.all(np.diff(n) <= 1e-13 * n[:-1])
    Z2 = oracle.path_walk(q, w, np.full(T, 2.0), T - 1, lib=lib)
    n2 = np.linalg.norm(Z2, axis=1)
    np.testing.assert_allclose(n2, n2[0], rtol=1e-13)
    Z1 = oracle.path_walk(q, w, np.full(T, 1.0), T - 1, lib=lib)
    # Z1[m] = H_{T-m} ... H_{T-1} q: the last factor applied is H_{T-m}
    for m in range(1, T):
        t = T - m
        assert abs(w[t] @ Z1[m]) <= 1e-13 * (1 + np.linalg.norm(Z1[m]))
    # a different beta_t gives a different walk (the update is not dropped)
    assert np.max(np.abs(Z[-1] - q[T - 1])) > 1e-3


def pin_first_token_factors_unused(lib):
    """H_0 and f_0 never enter a logit (the product starts at H_{j+1}, j >= 0):
    outputs are bitwise invariant to w_0, beta_0 and log f_0."""
    rng = np.random.default_rng(110)
    T, d = 24, 8
    q, k, v, w, beta = _rand_inputs(rng, T, d)
    logf = -rng.uniform(0.0, 0.5, size=T)
    o1, l1 = oracle.path_attn(q, k, v, w, beta, logf, lib=lib)
    w2, b2, f2 = w.copy(), beta.copy(), logf.copy()
    w2[0] = rng.standard_normal(d)
    b2[0] = 1.234
    f2[0] = -3.0
    o2, l2 = oracle.path_attn(q, k, v, w2, b2, f2, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # ... but w_1 does enter (row 1 against key 0)
    w3 = w.copy()
    w3[1] = -w3[2]
    o3, _ = oracle.path_attn(q, k, v, w3, beta, logf, lib=lib)
    assert not np.array_equal(o1[1], o3[1])


def pin_first_row(lib):
    """Row 0 attends only to key 0: o_0 = v_0 and lse_0 = scale q_0 . k_0."""
    rng = np.random.default_rng(111)
    T, d = 8, 8
    q, k, v, w, beta = _rand_inputs(rng, T, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle.path_attn(q, k, v, w, beta, scale=scale, lib=lib)
    assert np.array_equal(o[0], v[0])
    assert abs(lse[0] - scale * (q[0] @ k[0])) <= 1e-15 * (1 + abs(lse[0]))


def pin_zero_gate_is_plain(lib):
    """log f = 0 (f = 1, nothing forgotten) gives plain PaTH exactly."""
    rng = np.random.default_rng(112)
    T, d = 20, 8
    q, k, v, w, beta = _rand_inputs(rng, T, d)
    o1, l1 = oracle.path_attn(q, k, v, w, beta, None, lib=lib)
    o2, l2 = oracle.path_attn(q, k, v, w, beta, np.zeros(T), lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_rows_api_matches_full(lib):
    """The row-sampling entry returns the same values as the full pass, with
    several heads and out-of-order rows."""
    rng = np.random.default_rng(113)
    nh, T, d = 3, 20, 4
    q = rng.standard_normal((nh, T, d))
    k = rng.standard_normal((nh, T, d))
    v = rng.standard_normal((nh, T, d))
    w = rng.standard_normal((nh, T, d))
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = rng.uniform(0, 2, size=(nh, T))
    o, lse = oracle.path_attn(q, k, v, w, beta, lib=lib)
    rows = np.array([[2, 19], [0, 0], [1, 7], [2, 3]])
    o_r, l_r = oracle.path_attn_rows(q, k, v, w, beta, None, 0.5, rows, lib=lib)
    for r, (h, i) in enumerate(rows):
        o_h, l_h = oracle.path_attn(q[h], k[h], v[h], w[h], beta[h], scale=0.5, lib=lib)
        assert np.array_equal(o_r[r], o_h[i]) and l_r[r] == l_h[i]
    # head separation: head 1 of the batched call equals a single-head call
    o1, l1 = oracle.path_attn(q[1], k[1], v[1], w[1], beta[1], lib=lib)
    assert np.array_equal(o[1], o1) and np.array_equal(lse[1], l1)


ALL_PINS = [
    pin_beta0_is_causal_attention,
    pin_beta0_fox_is_forgetting_attention,
    pin_swap_closed_form,
    pin_swap_golden,
    pin_dense_products,
    pin_linear_rnn,
    pin_decode_key_refinement,
    pin_global_ut_formula,
    pin_chunked_algorithm,
    pin_chunk_quantities,
    pin_softmax_readout,
    pin_eigen_direction_golden,
    pin_walk_invariants,
    pin_first_token_factors_unused,
    pin_first_row,
    pin_zero_gate_is_plain,
    pin_rows_api_matches_full,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__[4:])
def test_oracle_pin(pin):
    pin(oracle.load())


def test_partial_path_splits_into_path_and_plain_dot():
    """Partial PaTH (the position transform acting on a subspace): with
    w_t zero on the last coordinates, every H_t is the identity there, so the
    path logit is the PaTH logit of the leading coordinates plus the ordinary
    dot product of the trailing ones."""
    rng = np.random.default_rng(501)
    T, dp, dn = 23, 4, 3
    q, k = rng.standard_normal((T, dp + dn)), rng.standard_normal((T, dp + dn))
    w = np.zeros((T, dp + dn))
    w[:, :dp] = rng.standard_normal((T, dp))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    beta = rng.uniform(0.0, 2.0, size=T)
    S = oracle.path_logits(q, k, w, beta)
    S_p = oracle.path_logits(q[:, :dp], k[:, :dp], w[:, :dp], beta)
    plain = q[:, dp:] @ k[:, dp:].T
    low = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(S[low], (S_p + plain)[low], rtol=1e-12, atol=1e-12)
