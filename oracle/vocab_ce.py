"""fp64 oracle of the linear-head cross-entropy over a large vocabulary.

Test infrastructure only: the tests, the smoke check and the bench's CPU
baseline call it; the product path never does, and it shares no code with the
HIP kernels (both sides import only the seeded input generator).

What is computed follows two passages. rwkv-metal, "Open problems /
contributions welcome", asks for a loss over the World vocabulary (65536) that
streams over the vocabulary instead of materialising the [B*T, vocab] logits:
an online softmax in the forward and softmax-form gradients in the backward.
rwkv-lab, "From-scratch pretraining lab" (file table), names a fused LM-head
cross-entropy with pad masking. Neither prints a formula; this is the
textbook definition of the per-row cross-entropy of a linear head, written
out on the dense logits (the plain definition the streaming kernel must reach
up to rounding order):

    z[m, v]   = sum_d h[m, d] W[v, d]
    lse[m]    = log sum_v exp(z[m, v])
    loss[m]   = lse[m] - z[m, t_m]                    (0 for a masked row)
    G[m, v]   = dloss[m] (exp(z[m, v] - lse[m]) - [v == t_m])   (0 for a masked row)
    dh        = G W          dW = G^T h

A row is masked (a pad row) when its target is outside [0, V); callers put an
ignore index such as -100 there. lse is returned for every row.

Shapes: h [M, D], W [V, D], targets [M] integers, dloss [M]. All arithmetic
is fp64.
"""
from __future__ import annotations

import numpy as np


def _d(x):
    return np.asarray(x, dtype=np.float64)


def valid_rows(targets, V):
    t = np.asarray(targets).astype(np.int64)
    return (t >= 0) & (t < V)


def logits(h, W):
    """z = h W^T, [M, V]."""
    return _d(h) @ _d(W).T


def logsumexp_rows(z):
    """log sum_v exp(z[m, v]) with the row maximum taken out first."""
    zmax = z.max(axis=1, keepdims=True)
    return (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))[:, 0]


def forward(h, W, targets):
    """Returns (loss [M], lse [M])."""
    V = np.shape(W)[0]
    z = logits(h, W)
    lse = logsumexp_rows(z)
    ok = valid_rows(targets, V)
    t = np.where(ok, np.asarray(targets).astype(np.int64), 0)
    zt = z[np.arange(z.shape[0]), t]
    loss = np.where(ok, lse - zt, 0.0)
    return loss, lse


def grad_logits(h, W, targets, dloss):
    """G [M, V] = dloss (softmax(z) - onehot(t)), zero rows where masked."""
    V = np.shape(W)[0]
    z = logits(h, W)
    lse = logsumexp_rows(z)
    p = np.exp(z - lse[:, None])
    ok = valid_rows(targets, V)
    rows = np.nonzero(ok)[0]
    p[rows, np.asarray(targets).astype(np.int64)[rows]] -= 1.0
    p *= _d(dloss)[:, None]
    p[~ok] = 0.0
    return p


def backward(h, W, targets, dloss):
    """Returns (dh [M, D], dW [V, D]) of sum_m dloss[m] loss[m]."""
    G = grad_logits(h, W, targets, dloss)
    return G @ _d(W), G.T @ _d(h)
