"""fp64 gradients of PaTH attention -- test infrastructure only (imported by
``tests/`` alone; nothing in the HIP path imports it, and it imports nothing
from the HIP path).

The forward pass is the definition of the PaTH slides for arXiv:2505.16381v2,
frame "PaTH inserts a learned transformation along every path" (paper Sec.
2.2), with the forget gate of frame "FoX adds a separate mechanism for
forgetting":

    c_ij = k_j^T H_{j+1} ... H_i q_i,   H_t = I - beta_t w_t w_t^T   (j <= i)
    s_ij = scale * c_ij + sum_{s=j+1..i} log f_s,   o_i = sum_j softmax_j(s_ij) v_j

written here as plain PyTorch CPU float64 operations so that autograd gives
the exact gradients of a scalar loss <dO, o> + <dlse, lse>.  The logits are
formed by the right-to-left walk of the definition, vectorised over queries:
all query rows are carried together, and at key position j every row i >= j
first takes its logit against k_j and then crosses H_j (rows i < j have not
started their walk and stay untouched).  Nothing is blocked or reordered
beyond that.

Pins (tests/test_oracle_backward.py): the forward equals the C oracle; the
gradients equal central finite differences of the C oracle along random
directions; with beta = 0 they equal the textbook softmax-attention
gradients and the gradient of w vanishes.
"""
from __future__ import annotations

import numpy as np
import torch


def _logits(q, k, w, beta):
    """Raw path logits c [T, T] (j <= i; -inf above the diagonal) of one
    head; q, k, w [T, d], beta [T] float64 tensors."""
    T = q.shape[0]
    z = q.clone()                      # row i: q_i transported down to j
    rows = torch.arange(T)
    cols = []
    for j in range(T - 1, -1, -1):
        cols.append(z @ k[j])          # logit of every row against key j
        if j > 0:                      # cross H_j, rows i >= j only
            active = (rows >= j).to(z.dtype)[:, None]
            z = z - active * beta[j] * (z @ w[j])[:, None] * w[j][None, :]
    c = torch.stack(cols[::-1], dim=1)  # [i, j]
    mask = rows[None, :] <= rows[:, None]
    return torch.where(mask, c, torch.full_like(c, -torch.inf))


def forward(q, k, v, w, beta, logf=None, scale=None):
    """Outputs and lse of one head (float64 tensors, differentiable)."""
    T, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    s = scale * _logits(q, k, w, beta)
    if logf is not None:
        # Lambda_t = sum_{1<=s<=t} log f_s; f_0 enters no logit
        lam = torch.cat([logf.new_zeros(1), torch.cumsum(logf[1:], 0)])
        s = s + (lam[:, None] - lam[None, :])
    lse = torch.logsumexp(s, dim=1)
    p = torch.exp(s - lse[:, None])
    return p @ v, lse


def gradients(q, k, v, w, beta, logf, do, dlse=None, scale=None):
    """Gradients of <do, o> + <dlse, lse> for one head.  Arguments are numpy
    arrays ([T, d] and [T]); returns a dict of float64 numpy arrays dq, dk,
    dv, dw, dbeta and dlogf (None without the gate)."""
    t = lambda x: None if x is None else torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    tq, tk, tv, tw, tb, tf = t(q), t(k), t(v), t(w), t(beta), t(logf)
    o, lse = forward(tq, tk, tv, tw, tb, tf, scale)
    loss = (o * torch.tensor(np.asarray(do, dtype=np.float64))).sum()
    if dlse is not None:
        loss = loss + (lse * torch.tensor(np.asarray(dlse, dtype=np.float64))).sum()
    loss.backward()
    # an input the loss does not depend on (w, beta, log f when T = 1: H_0 and
    # f_0 enter no logit) has no .grad; its gradient is exactly zero
    g = lambda x: None if x is None else (x.grad.numpy().copy() if x.grad is not None
                                          else np.zeros(tuple(x.shape)))
    return dict(dq=g(tq), dk=g(tk), dv=g(tv), dw=g(tw), dbeta=g(tb), dlogf=g(tf),
                o=o.detach().numpy(), lse=lse.detach().numpy())
