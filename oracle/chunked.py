"""fp64 numpy statement of the blockwise algorithm -- oracle, test infrastructure.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares nothing with the HIP library.

Written from the PaTH discussion slides, frames "A triangular representation
makes paths computable", "A right-to-left scan accumulates cross-block paths"
and the backup frame "Backup: fix orientation before implementing UT products"
(paper Secs. 3.1-3.3).  For one chunk of C tokens with rows w_t^T stacked in W
and D = diag(beta):

    U   = (I + strictLower(D W W^T))^{-1} D                  (lower triangular)
    <-Q = Q - lower(Q W^T) U W          row i: (H_first ... H_i q_i)^T
    ->K = K - (U strictLower(W K^T))^T W   row j: (H_last ... H_{j+1} k_j)^T
    M   = W^T U W                       F^T = I - M, F = H_first ... H_last
    Al  = lower(Q K^T) - lower(Q W^T) U strictLower(W K^T)   (diagonal block)

and the cross-chunk logits of query chunk b against key chunk c < b are
Q_work ->K_c^T, with Q_work = <-Q_b and Q_work <- Q_work (I - M_c) after each
key chunk.  The oracle pins check that this algebra reproduces the plain
definition (oracle/path_oracle.c) for several chunk sizes; the GPU tests use
``chunk_quantities`` as the reference for the chunk-preparation outputs.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_quantities(Q, K, W, beta):
    """Prep quantities of one chunk (all fp64): U, Qa(<-Q), Kb(->K), M, Al."""
    C = W.shape[0]
    D = np.diag(beta)
    N = np.tril(D @ W @ W.T, -1)
    U = solve_triangular(np.eye(C) + N, D, lower=True, unit_diagonal=True)
    QW = np.tril(Q @ W.T)
    WK = np.tril(W @ K.T, -1)
    Qa = Q - QW @ U @ W
    Kb = K - (U @ WK).T @ W
    M = W.T @ U @ W
    Al = np.tril(Q @ K.T) - QW @ U @ WK
    return U, Qa, Kb, M, Al


def chunked_logits(q, k, w, beta, C):
    """Raw (unscaled, ungated) causal logits [T, T] of one head via the
    blockwise right-to-left scan; -inf above the diagonal."""
    T, d = q.shape
    assert T % C == 0
    n = T // C
    parts = [chunk_quantities(q[c * C:(c + 1) * C], k[c * C:(c + 1) * C],
                              w[c * C:(c + 1) * C], beta[c * C:(c + 1) * C])
             for c in range(n)]
    A = np.full((T, T), -np.inf)
    for b in range(n):
        _, Qa, _, _, Al = parts[b]
        rb = slice(b * C, (b + 1) * C)
        blk = np.where(np.tril(np.ones((C, C), dtype=bool)), Al, -np.inf)
        A[rb, rb] = blk
        Qw = Qa.copy()
        for c in range(b - 1, -1, -1):
            _, _, Kb, M, _ = parts[c]
            A[rb, c * C:(c + 1) * C] = Qw @ Kb.T
            Qw = Qw - Qw @ M
    return A
