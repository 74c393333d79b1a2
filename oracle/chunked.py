"""fp64 numpy statement of the blockwise quantities -- oracle, test infrastructure.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares nothing with the HIP library.

Two things are stated here, each from the PaTH discussion slides for
arXiv:2505.16381v2 (paper Secs. 3.1-3.3):

* ``chunk_quantities``: what the chunk preparation produces, from the
  definitions, as explicit products of the d x d factors H_t = I - beta_t w_t
  w_t^T of one chunk (t = first .. last):
      <-Q row i = H_first ... H_i q_i            (the query moved to the chunk start)
      ->K row j = H_last ... H_{j+1} k_j         (the key moved to the chunk end)
      F         = H_first ... H_last,  M = I - F^T
      Al[i, j]  = k_j^T H_{j+1} ... H_i q_i      (j <= i, the diagonal block)
  (frame "A right-to-left scan accumulates cross-block paths" names <-Q, ->K
  and F; its footnote fixes F's orientation.)

* ``ut_chunk_quantities``: the same four quantities by the shared matrix
  operations of frames "A triangular representation makes paths computable"
  and "Backup: fix orientation before implementing UT products":
      U   = (I + strictLower(D W W^T))^{-1} D      (library triangular solve)
      <-Q = Q - lower(Q W^T) U W
      ->K = K - (U strictLower(W K^T))^T W
      M   = W^T U W
      Al  = lower(Q K^T) - lower(Q W^T) U strictLower(W K^T).
  tests/test_oracle_pins.py pins the two against each other and both against
  the walk of the definition.

``chunked_logits`` runs the scan of frame "A right-to-left scan accumulates
cross-block paths" one query row at a time: the row's diagonal-block logits
come from Al; its moved query z = <-Q row starts at its chunk's first token
and, for each earlier chunk c (nearest first), is first dotted with every key
of c (->K_c z) and then carried across the chunk, z <- F_c z.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _factors(W, beta):
    d = W.shape[1]
    return [np.eye(d) - beta[t] * np.outer(W[t], W[t]) for t in range(W.shape[0])]


def chunk_quantities(Q, K, W, beta):
    """Per-chunk quantities of one chunk (fp64) from their definitions.

    Returns a dict with qa (<-Q, [C, d]), kb (->K, [C, d]), F (H_first ...
    H_last, [d, d]), m (I - F^T) and al ([C, C]; entries above the diagonal
    are -inf)."""
    C, d = W.shape
    H = _factors(W, beta)
    qa = np.empty((C, d))
    al = np.full((C, C), -np.inf)
    for i in range(C):
        z = np.array(Q[i], dtype=np.float64)
        for t in range(i, -1, -1):          # read key t, then cross H_t
            al[i, t] = K[t] @ z
            z = H[t] @ z
        qa[i] = z                           # H_first ... H_i q_i
    kb = np.empty((C, d))
    for j in range(C):
        z = np.array(K[j], dtype=np.float64)
        for t in range(j + 1, C):
            z = H[t] @ z
        kb[j] = z                           # H_last ... H_{j+1} k_j
    F = np.eye(d)
    for t in range(C):
        F = F @ H[t]                        # H_first ... H_last
    return dict(qa=qa, kb=kb, F=F, m=np.eye(d) - F.T, al=al)


def ut_chunk_quantities(Q, K, W, beta):
    """The same quantities by the UT form (fp64): dict with U, qa, kb, m and
    al (al only on and below the diagonal)."""
    C = W.shape[0]
    D = np.diag(beta)
    U = solve_triangular(np.eye(C) + np.tril(D @ W @ W.T, -1), D, lower=True,
                         unit_diagonal=True)
    QW = np.tril(Q @ W.T)
    WK = np.tril(W @ K.T, -1)
    return dict(U=U, qa=Q - QW @ U @ W, kb=K - (U @ WK).T @ W, m=W.T @ U @ W,
                al=np.tril(Q @ K.T) - QW @ U @ WK)


def chunked_logits(q, k, w, beta, C):
    """Raw (unscaled, ungated) causal logits [T, T] of one head via the
    blockwise right-to-left scan, row by row; -inf above the diagonal."""
    T, d = q.shape
    assert T % C == 0
    n = T // C
    sl = lambda c: slice(c * C, (c + 1) * C)
    parts = [chunk_quantities(q[sl(c)], k[sl(c)], w[sl(c)], beta[sl(c)]) for c in range(n)]
    A = np.full((T, T), -np.inf)
    for i in range(T):
        b, r = divmod(i, C)
        A[i, b * C:b * C + r + 1] = parts[b]["al"][r, :r + 1]
        z = parts[b]["qa"][r].copy()
        for c in range(b - 1, -1, -1):      # nearest earlier chunk first
            A[i, sl(c)] = parts[c]["kb"] @ z  # read chunk c ...
            z = parts[c]["F"] @ z             # ... then cross its transition
    return A
