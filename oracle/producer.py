"""fp64 numpy statement of the w / beta producer -- oracle, test infrastructure.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares nothing with the HIP library.

What it computes (PaTH slides for arXiv:2505.16381v2, frame "PaTH inserts a
learned transformation along every path": beta_t = 2 sigmoid(u^T x_t + b),
||w_t||_2 = 1, and w_t produced by a low-rank projection, a convolution of
width 3 and an L2 normalisation; the authors' discussion page, section "Model
Architecture Details": linear projection, short convolution, L2
normalisation per head, the projection low-rank in the manner of LoRA), for
hidden states x of shape [B, T, Dm] and H heads of size d:

    z_t    = Wu (Wd x_t)                          Wd: [R, Dm],  Wu: [H d, R]
    z'_t   = cw[:, 0] * z_{t-2} + cw[:, 1] * z_{t-1} + cw[:, 2] * z_t
             (per channel, causal; z_t = 0 for t < 0)
    w_t[h] = z'_t[h d : (h + 1) d] / || z'_t[h d : (h + 1) d] ||_2
             (a zero vector gives w = 0, so that H_t = I)
    beta_t[h] = 2 sigmoid(u[h] . x_t + ub[h])     u: [H, Dm]

Readings where the pages are silent: no bias in the projections, no
activation after the convolution, the taps ordered oldest first, weights
stored output-major ([out, in]).  Outputs: w as [B, H, T, d], beta as
[B, H, T].  Parity is pinned by tests/test_oracle_producer.py (unit norms,
locality of the convolution, scale and sign behaviour of the normalisation,
closed forms of beta, a hand-worked example).
"""
from __future__ import annotations

import numpy as np


def producer(x, Wd, Wu, cw, u, ub, H: int, d: int):
    """w [B, H, T, d] and beta [B, H, T] in float64 from the definitions above."""
    x = np.asarray(x, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    Wu = np.asarray(Wu, dtype=np.float64)
    cw = np.asarray(cw, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    ub = np.asarray(ub, dtype=np.float64)
    B, T, Dm = x.shape
    assert Wd.shape[1] == Dm and Wu.shape == (H * d, Wd.shape[0])
    assert cw.shape == (H * d, 3) and u.shape == (H, Dm) and ub.shape == (H,)
    # low-rank projection, token by token
    z = np.einsum("btm,rm->btr", x, Wd)
    z = np.einsum("btr,cr->btc", z, Wu)                 # [B, T, H d]
    # causal convolution of width 3 along the tokens
    zc = np.zeros_like(z)
    for t in range(T):
        for k in range(3):
            s = t - 2 + k
            if s >= 0:
                zc[:, t, :] += cw[:, k] * z[:, s, :]
    # L2 normalisation per head
    zc = zc.reshape(B, T, H, d)
    nrm = np.sqrt(np.sum(zc * zc, axis=-1, keepdims=True))
    w = np.where(nrm > 0.0, zc / np.where(nrm > 0.0, nrm, 1.0), 0.0)
    w = np.transpose(w, (0, 2, 1, 3))                   # [B, H, T, d]
    logit = np.einsum("btm,hm->bht", x, u) + ub[None, :, None]
    beta = 2.0 / (1.0 + np.exp(-logit))
    return w, beta
