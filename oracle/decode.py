"""fp64 statement of PaTH decoding with in-place key refinement -- test
infrastructure only (imported by ``tests/`` alone; nothing in the HIP path
imports it, and it imports nothing from the HIP path).

PaTH discussion slides for arXiv:2505.16381v2, frame "Decoding updates
historical keys in place" (paper Sec. 3.4, Eq. (1)): when token t arrives,
every earlier cached key is reflected by H_t = I - beta_t w_t w_t^T,

    k_j^(t) = k_j^(t-1) - beta_t w_t (w_t^T k_j^(t-1)),   j < t,

so that (k_j^(t))^T q_t = k_j^T H_{j+1} ... H_t q_t, the path logit, and the
readout is ordinary softmax attention over the refined keys.  Before decoding,
the cache of a prompt of length L holds every key aligned to the prompt end:
k_j^(L-1) = H_{L-1} ... H_{j+1} k_j.

The functions below are that definition written out (a loop over t applying
one reflection at a time); the decoded outputs themselves are rows of the
forward oracle (``oracle.path_attn_rows``), since a decode step at position t
computes exactly row t of the attention.

Pins (tests/test_oracle_pins.py): refined keys dotted with q_i reproduce the
independently pinned logit oracle; beta = 0 leaves keys unchanged; with exact
unit w and beta = 2 every refinement is a reflection and preserves norms.
"""
from __future__ import annotations

import numpy as np


def refined_keys(k, w, beta, upto: int):
    """Keys of one head aligned to position `upto`: row j (j <= upto) is
    H_upto ... H_{j+1} k_j, fp64.  k, w: [T, d]; beta: [T].  Returns
    [upto + 1, d].  Applies H_t for t = 1 .. upto in order, each to the keys
    that precede t, exactly as the decoding recurrence does."""
    k = np.array(k[: upto + 1], dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    for t in range(1, upto + 1):
        prev = k[:t]
        prev -= beta[t] * np.outer(prev @ w[t], w[t])
    return k


def aligned_key_rows(k, w, beta, rows, upto: int):
    """Selected keys of one head aligned to position `upto`: for each j in
    `rows` (j <= upto), H_upto ... H_{j+1} k_j, fp64, obtained by applying
    H_{j+1}, H_{j+2}, ..., H_upto to k_j one reflection at a time.  k, w:
    [T, d]; beta: [T].  Returns [len(rows), d].  Cost O((upto - j) d) per
    row, so full-length contexts can be sampled."""
    w = np.asarray(w, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    out = []
    for j in rows:
        z = np.array(k[j], dtype=np.float64)
        for t in range(j + 1, upto + 1):
            z -= beta[t] * (w[t] @ z) * w[t]
        out.append(z)
    return np.stack(out) if out else np.zeros((0, np.shape(k)[-1]))


def gate_prefix(logf):
    """Lambda_t = sum_{s=1..t} log f_s (fp64; f_0 never enters a logit).
    logf: [..., T]."""
    logf = np.asarray(logf, dtype=np.float64)
    lam = np.cumsum(logf, axis=-1)
    return lam - logf[..., :1]
