"""Pins of the vocabulary cross-entropy oracle (oracle/vocab_ce.py) to facts
that do not come from the oracle itself: closed forms (uniform logits, the
two-class logistic case), a library routine for the same special function
(scipy's log_softmax / logsumexp), invariances (a per-row logit shift, a
permutation of the vocabulary), exact gradient identities, fp64 central
finite differences, and the large-logit limit. Each pin returns an error
that must stay within its tolerance."""
import numpy as np
import pytest
import scipy.special as sp

from linear_recurrent_lm_amd import synth
from oracle import vocab_ce as V


def _inputs(M, D, Vn, seed, dloss="normal", pad_frac=0.2):
    c = synth.make_ce_inputs(M, D, Vn, seed=seed, pad_frac=pad_frac, dloss=dloss)
    return c.h.astype(np.float64), c.W.astype(np.float64), c.targets, c.dloss.astype(np.float64)


def _rel(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def pin_uniform_logits(seed=51):
    """W = 0: every logit is 0, lse = log V, loss = log V on unmasked rows,
    G = dloss (1/V - onehot), dh = 0 and dW[v] = (1/V) sum_m dloss_m h_m
    - sum_{m: t_m = v} dloss_m h_m."""
    h, W, t, dl = _inputs(13, 24, 37, seed)
    W = np.zeros_like(W)
    loss, lse = V.forward(h, W, t)
    ok = (t >= 0) & (t < 37)
    err = max(_rel(lse, np.full(13, np.log(37.0))),
              _rel(loss, np.where(ok, np.log(37.0), 0.0)))
    dh, dW = V.backward(h, W, t, dl)
    want = np.tile((dl[ok, None] * h[ok]).sum(axis=0) / 37.0, (37, 1))
    for m in np.nonzero(ok)[0]:
        want[t[m]] -= dl[m] * h[m]
    return max(err, float(np.max(np.abs(dh))), _rel(dW, want))


def pin_logistic_two_classes(seed=52):
    """V = 2: loss = softplus(z_o - z_t) = -log sigmoid(z_t - z_o), and the
    gradients are sigmoid(z_o - z_t) (W_o - W_t) for h, +/- sigmoid(z_o - z_t) h
    for the two rows of W (each row weighted by dloss)."""
    h, W, t, dl = _inputs(11, 16, 2, seed, pad_frac=0.0)
    loss, _ = V.forward(h, W, t)
    dh, dW = V.backward(h, W, t, dl)
    want_loss = np.empty(11)
    want_dh = np.empty_like(h)
    want_dW = np.zeros_like(W)
    for m in range(11):
        o = 1 - t[m]
        zt = float(np.dot(h[m], W[t[m]]))
        zo = float(np.dot(h[m], W[o]))
        want_loss[m] = -sp.log_expit(zt - zo)
        s = sp.expit(zo - zt)
        want_dh[m] = dl[m] * s * (W[o] - W[t[m]])
        want_dW[o] += dl[m] * s * h[m]
        want_dW[t[m]] -= dl[m] * s * h[m]
    return max(_rel(loss, want_loss), _rel(dh, want_dh), _rel(dW, want_dW))


def pin_scipy_log_softmax(seed=53):
    """loss = -log_softmax(z)[t] and lse = logsumexp(z), from scipy."""
    h, W, t, dl = _inputs(17, 32, 300, seed)
    loss, lse = V.forward(h, W, t)
    z = np.einsum("md,vd->mv", h, W)
    ls = sp.log_softmax(z, axis=1)
    ok = (t >= 0) & (t < 300)
    want = np.where(ok, -ls[np.arange(17), np.where(ok, t, 0)], 0.0)
    return max(_rel(loss, want), _rel(lse, sp.logsumexp(z, axis=1)))


def pin_shift_invariance(seed=54):
    """A per-row constant c_m added to every logit (an extra feature c_m
    against an all-ones column of W) raises lse by c_m and leaves the loss and
    the gradients of the original columns unchanged."""
    h, W, t, dl = _inputs(9, 16, 50, seed)
    c = np.random.Generator(np.random.PCG64(seed)).normal(0, 30, size=9)
    h2 = np.concatenate([h, c[:, None]], axis=1)
    W2 = np.concatenate([W, np.ones((50, 1))], axis=1)
    l1, s1 = V.forward(h, W, t)
    l2, s2 = V.forward(h2, W2, t)
    dh1, dW1 = V.backward(h, W, t, dl)
    dh2, dW2 = V.backward(h2, W2, t, dl)
    return max(_rel(l2, l1), _rel(s2 - c, s1), _rel(dh2[:, :16], dh1), _rel(dW2[:, :16], dW1))


def pin_vocab_permutation(seed=55):
    """Relabelling the vocabulary (rows of W and the targets) permutes dW and
    changes nothing else."""
    h, W, t, dl = _inputs(10, 8, 40, seed)
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(40)
    inv = np.argsort(perm)
    t2 = np.where((t >= 0) & (t < 40), inv[np.clip(t, 0, 39)], t)
    l1, s1 = V.forward(h, W, t)
    l2, s2 = V.forward(h, W[perm], t2)
    dh1, dW1 = V.backward(h, W, t, dl)
    dh2, dW2 = V.backward(h, W[perm], t2, dl)
    return max(_rel(l2, l1), _rel(s2, s1), _rel(dh2, dh1), _rel(dW2, dW1[perm]))


def pin_gradient_identities(seed=56):
    """Each unmasked row of G sums to zero, so sum_v dW[v] = 0; masked rows
    have zero loss and zero dh and do not reach dW (changing their h leaves dW
    unchanged)."""
    h, W, t, dl = _inputs(21, 12, 33, seed, pad_frac=0.3)
    dh, dW = V.backward(h, W, t, dl)
    loss, _ = V.forward(h, W, t)
    bad = ~((t >= 0) & (t < 33))
    assert bad.any()
    h2 = h.copy()
    h2[bad] += 5.0
    _, dW2 = V.backward(h2, W, t, dl)
    scale = float(np.max(np.abs(dW)))
    return max(float(np.max(np.abs(dW.sum(axis=0)))) / scale,
               float(np.max(np.abs(loss[bad]))), float(np.max(np.abs(dh[bad]))),
               _rel(dW2, dW))


def pin_finite_differences(seed=57, eps=1e-6):
    """dh and dW against central differences of sum_m dloss_m loss_m."""
    h, W, t, dl = _inputs(6, 5, 9, seed)
    dh, dW = V.backward(h, W, t, dl)
    f = lambda hh, WW: float(np.dot(dl, V.forward(hh, WW, t)[0]))
    err = 0.0
    for (x, g, is_h) in ((h, dh, True), (W, dW, False)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num = (f(xp, W) - f(xm, W)) if is_h else (f(h, xp) - f(h, xm))
            err = max(err, abs(num / (2 * eps) - g[idx]))
    return err / max(float(np.max(np.abs(dh))), float(np.max(np.abs(dW))))


def pin_large_logits(seed=58, s=1e4):
    """Logits of size 1e4 stay finite, and as the logits grow by a factor s the
    loss approaches s (max_v z_v - z_t): the gap is at most log V."""
    h, W, t, dl = _inputs(8, 16, 64, seed, pad_frac=0.0)
    loss, lse = V.forward(h, s * W, t)
    z = h @ W.T
    want = s * (z.max(axis=1) - z[np.arange(8), t])
    gap = np.abs(loss - want)
    ok = np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    return float(np.max(gap)) / np.log(64.0) if ok else np.inf


def pin_dloss_linearity(seed=59):
    """The gradients are linear in dloss."""
    h, W, t, d1 = _inputs(7, 8, 20, seed)
    d2 = np.random.Generator(np.random.PCG64(seed)).standard_normal(7)
    a = V.backward(h, W, t, d1 + 2.0 * d2)
    b1 = V.backward(h, W, t, d1)
    b2 = V.backward(h, W, t, d2)
    return max(_rel(a[0], b1[0] + 2 * b2[0]), _rel(a[1], b1[1] + 2 * b2[1]))


PINS = {
    "uniform_logits": (pin_uniform_logits, 1e-12),
    "logistic_two_classes": (pin_logistic_two_classes, 1e-12),
    "scipy_log_softmax": (pin_scipy_log_softmax, 1e-12),
    "shift_invariance": (pin_shift_invariance, 1e-10),
    "vocab_permutation": (pin_vocab_permutation, 1e-12),
    "gradient_identities": (pin_gradient_identities, 1e-12),
    "finite_differences": (pin_finite_differences, 1e-6),
    "large_logits": (pin_large_logits, 1.0),
    "dloss_linearity": (pin_dloss_linearity, 1e-12),
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_vce_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, (name, err)
