"""fp64 statement of the blockwise backward pass -- oracle, test infrastructure
(only tests/ import it; it shares nothing with the HIP library).

The pages give no backward algorithm; this module states, in plain fp64
numpy, the blockwise decomposition the GPU path computes, so that each of its
intermediate quantities can be checked on its own.  It is pinned to
oracle/backward.py (autograd of the definition) in
tests/test_oracle_backward.py: the final gradients must agree, for small
chunk sizes and at the chunk length 64 with head dims 64 and 128 (the sizes at
which the GPU tests use it).

Forward algebra (oracle/chunked.py, ut_chunk_quantities; PaTH slides, frames "A triangular
representation makes paths computable", "A right-to-left scan accumulates
cross-block paths", "Backup: fix orientation before implementing UT
products"): per chunk c, Qa = <-Q_c, Kb = ->K_c, M_c, Al_c.  Keys of chunks
before c aligned to the start of chunk c ("key levels", the decoding view of
frame "Decoding updates historical keys in place") satisfy

    Khat[0] = (empty),   Khat[c+1] = [ Khat[c] (I - M_c)^T ; Kb_c ],

and the cross logits of query chunk c are Qa_c Khat[c]^T.

Backward: with g = scale * dS the gradient of the raw logits,
    dQa_c = g Khat[c],   dV[j] += P^T dO_c,   Gamma += g^T Qa_c,
where Gamma is the gradient of Khat[c] accumulated over query chunks >= c.
Crossing from c down to c - 1 (Khat[c] = [Khat[c-1] (I - M_{c-1})^T ; Kb_{c-1}]):
    dKb_{c-1} = Gamma[rows of chunk c-1],
    dM_{c-1}  = -Gamma[rows < chunk c-1]^T Khat[c-1],
    Gamma     <- Gamma[rows < chunk c-1] (I - M_{c-1}).
Finally each chunk's (dQa, dKb, dM, dAl) is mapped to (dq, dk, dw, dbeta)
through the UT formulas (chunk_vjp), and the forget gate's Lambda gradient to
log f by suffix sums.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.chunked import ut_chunk_quantities


def _chunk_forward_torch(Q, K, W, beta):
    C = W.shape[0]
    D = torch.diag(beta)
    N = torch.tril(D @ W @ W.T, -1)
    U = torch.linalg.solve_triangular(torch.eye(C, dtype=W.dtype) + N, D, upper=False,
                                      unitriangular=True)
    QW = torch.tril(Q @ W.T)
    WK = torch.tril(W @ K.T, -1)
    Qa = Q - QW @ U @ W
    Kb = K - (U @ WK).T @ W
    M = W.T @ U @ W
    Al = torch.tril(Q @ K.T) - QW @ U @ WK
    return Qa, Kb, M, Al


def chunk_vjp(Q, K, W, beta, dQa, dKb, dM, dAl):
    """Gradients of one chunk's inputs (dQ, dK, dW, dbeta) given the
    gradients of its UT quantities (lower part of dAl used)."""
    t = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    tQ, tK, tW, tb = t(Q), t(K), t(W), t(beta)
    outs = _chunk_forward_torch(tQ, tK, tW, tb)
    gos = [torch.tensor(np.asarray(x, dtype=np.float64)) for x in (dQa, dKb, dM, np.tril(dAl))]
    grads = torch.autograd.grad(outs, (tQ, tK, tW, tb), gos)
    return [g.numpy() for g in grads]


def key_levels(Kb, M, C):
    """Khat[c] for c = 0..n-1 (list of [C*c, d] arrays)."""
    n = len(Kb)
    d = Kb[0].shape[1]
    lev = [np.zeros((0, d))]
    for c in range(n - 1):
        lev.append(np.concatenate([lev[c] @ (np.eye(d) - M[c]).T, Kb[c]], axis=0))
    return lev


def sweep_backward(q, k, v, w, beta, logf, do, o, lse, dlse=None, scale=None, C=64):
    """Blockwise gradients of <do, o> + <dlse, lse> for one head (fp64).

    o, lse: the forward outputs.  Returns a dict with the final gradients
    (dq, dk, dv, dw, dbeta, dlogf) and the intermediates (dQa, dKb, dM, dAl
    per chunk, the key levels)."""
    q, k, v, w, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, w, beta))
    do, o, lse = (np.asarray(x, dtype=np.float64) for x in (do, o, lse))
    T, d = q.shape
    assert T % C == 0
    n = T // C
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dl = np.zeros(T) if dlse is None else np.asarray(dlse, dtype=np.float64)
    if logf is not None:
        lf = np.asarray(logf, dtype=np.float64)
        lam = np.concatenate([[0.0], np.cumsum(lf[1:])])
    else:
        lam = np.zeros(T)
    sl = lambda c: slice(c * C, (c + 1) * C)
    parts = [ut_chunk_quantities(q[sl(c)], k[sl(c)], w[sl(c)], beta[sl(c)]) for c in range(n)]
    Qa = [p["qa"] for p in parts]
    Kb = [p["kb"] for p in parts]
    M = [p["m"] for p in parts]
    Al = [p["al"] for p in parts]
    lev = key_levels(Kb, M, C)
    Dv = np.sum(do * o, axis=1)

    dV = np.zeros((T, d))
    dLam = np.zeros(T)
    dQa = [None] * n
    dKb = [np.zeros((C, d)) for _ in range(n)]
    dM = [np.zeros((d, d)) for _ in range(n)]
    dAl = [None] * n
    Gam = np.zeros((C * (n - 1), d))
    low = np.tril(np.ones((C, C), dtype=bool))
    for c in range(n - 1, -1, -1):
        r = sl(c)
        # diagonal block
        sd = scale * Al[c] + (lam[r][:, None] - lam[r][None, :])
        pd = np.where(low, np.exp(np.where(low, sd, 0.0) - lse[r][:, None]), 0.0)
        dpd = do[r] @ v[r].T
        dsd = pd * (dpd - Dv[r][:, None] + dl[r][:, None])
        dAl[c] = scale * dsd
        dV[r] += pd.T @ do[r]
        dLam[r] += dsd.sum(1) - dsd.sum(0)
        # cross blocks against every earlier key, aligned to chunk c
        K_hat = lev[c]
        if c > 0:
            keys = slice(0, C * c)
            s = scale * Qa[c] @ K_hat.T + (lam[r][:, None] - lam[keys][None, :])
            p = np.exp(s - lse[r][:, None])
            dp = do[r] @ v[keys].T
            ds = p * (dp - Dv[r][:, None] + dl[r][:, None])
            g = scale * ds
            dV[keys] += p.T @ do[r]
            dLam[r] += ds.sum(1)
            dLam[keys] -= ds.sum(0)
            dQa[c] = g @ K_hat
            Gam[:C * c] += g.T @ Qa[c]
            # cross chunk c-1's transition downward
            dKb[c - 1] = Gam[C * (c - 1):C * c].copy()
            rest = Gam[:C * (c - 1)]
            dM[c - 1] = -rest.T @ lev[c - 1]
            Gam[:C * (c - 1)] = rest @ (np.eye(d) - M[c - 1])
        else:
            dQa[c] = np.zeros((C, d))
    dq = np.zeros((T, d)); dk = np.zeros((T, d)); dw = np.zeros((T, d)); db = np.zeros(T)
    for c in range(n):
        r = sl(c)
        gq, gk, gw, gb = chunk_vjp(q[r], k[r], w[r], beta[r], dQa[c], dKb[c], dM[c], dAl[c])
        dq[r], dk[r], dw[r], db[r] = gq, gk, gw, gb
    dlogf = None
    if logf is not None:
        dlogf = np.concatenate([[0.0], np.cumsum(dLam[::-1])[::-1][1:]])
    return dict(dq=dq, dk=dk, dv=dV, dw=dw, dbeta=db, dlogf=dlogf,
                dQa=dQa, dKb=dKb, dM=dM, dAl=dAl, levels=lev)
