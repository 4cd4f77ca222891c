"""Planted slips in a restatement of the vocabulary cross-entropy oracle: each
one is swapped in for oracle/vocab_ce.py and at least one pin of
test_vce_oracle_pins.py must fail for it, while the unslipped restatement
passes every pin. This shows the pins constrain the definition, not merely
agree with the oracle."""
import numpy as np
import pytest

from oracle import vocab_ce as V
from tests import test_vce_oracle_pins as P


def _restated(mut):
    def lse_of(z):
        if mut == "no_max_shift":
            return np.log(np.exp(z).sum(axis=1))
        zmax = z.max(axis=1, keepdims=True)
        s = np.log(np.exp(z - zmax).sum(axis=1))
        return s if mut == "max_not_added_back" else s + zmax[:, 0]

    def target(t, Vn):
        t = np.asarray(t).astype(np.int64)
        ok = (t >= 0) & (t < Vn)
        if mut == "target_off_by_one":
            t = np.where(ok, (t + 1) % Vn, t)
        return t, ok

    def forward(h, W, t):
        z = np.asarray(h, np.float64) @ np.asarray(W, np.float64).T
        lse = lse_of(z)
        tt, ok = target(t, z.shape[1])
        zt = z[np.arange(z.shape[0]), np.where(ok, tt, 0)]
        loss = lse - zt if mut == "masked_rows_kept" else np.where(ok, lse - zt, 0.0)
        return loss, lse

    def backward(h, W, t, dl):
        h = np.asarray(h, np.float64)
        W = np.asarray(W, np.float64)
        z = h @ W.T
        axis = 0 if mut == "softmax_over_rows" else 1
        p = np.exp(z - z.max(axis=axis, keepdims=True))
        p /= p.sum(axis=axis, keepdims=True)
        tt, ok = target(t, z.shape[1])
        rows = np.nonzero(ok)[0]
        sign = 1.0 if mut == "onehot_sign" else -1.0
        p[rows, tt[rows]] += sign
        if mut != "dloss_dropped":
            p *= np.asarray(dl, np.float64)[:, None]
        if mut != "masked_rows_kept":
            p[~ok] = 0.0
        dh = p @ W
        if mut == "dh_without_onehot":
            q = p.copy()
            q[rows, tt[rows]] -= sign * np.asarray(dl, np.float64)[rows]
            dh = q @ W
        return dh, p.T @ h

    return forward, backward


SLIPS = ["no_max_shift", "max_not_added_back", "target_off_by_one", "masked_rows_kept",
         "softmax_over_rows", "onehot_sign", "dloss_dropped", "dh_without_onehot"]


def _failed_pins():
    failed = []
    for name, (fn, tol) in P.PINS.items():
        try:
            with np.errstate(all="ignore"):
                err = fn()
        except Exception as e:  # a crash of a pin counts as a detection
            failed.append((name, repr(e)))
            continue
        if not err <= tol:
            failed.append((name, err))
    return failed


@pytest.mark.parametrize("mutation", SLIPS)
def test_ce_slip_is_caught(mutation, monkeypatch):
    fwd, bwd = _restated(mutation)
    monkeypatch.setattr(V, "forward", fwd)
    monkeypatch.setattr(V, "backward", bwd)
    assert _failed_pins(), f"no pin detects slip {mutation}"


def test_ce_restatement_passes_pins(monkeypatch):
    fwd, bwd = _restated("none")
    monkeypatch.setattr(V, "forward", fwd)
    monkeypatch.setattr(V, "backward", bwd)
    assert _failed_pins() == []
