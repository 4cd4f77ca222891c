"""Planted mistakes: each test compiles a copy of the oracle with one plausible
slip (wrong operand, wrong index, wrong state read, dropped term, misplaced
checkpoint) and checks that at least one pin of test_oracle_pins.py fails for
it. This shows the pins constrain the oracle, not merely agree with it."""
import os
import subprocess

import numpy as np

import pytest

from oracle import oracle as O
from tests import test_oracle_pins as P

MUTATIONS = {
    # forward (a conceptual slip is planted at every site that shares it,
    # i.e. in the forward and in the backward's own forward sweep)
    "a_term_reads_decayed_state": ("acc += S[i * N + j] * at[j];",
                                   "acc += S[i * N + j] * wt[j] * at[j];", 1),
    "a_and_b_swapped": ("sa[i] * bt[j] + vt[i] * kt[j];",
                        "sa[i] * at[j] + vt[i] * kt[j];", 2),
    "v_k_outer_transposed": ("sa[i] * bt[j] + vt[i] * kt[j];",
                             "sa[i] * bt[j] + vt[j] * kt[i];", 2),
    "y_reads_transposed_state": ("for (int j = 0; j < N; ++j) acc += S[i * N + j] * rt[j];",
                                 "for (int j = 0; j < N; ++j) acc += S[j * N + i] * rt[j];", 1),
    "decay_on_rows": ("S[i * N + j] = S[i * N + j] * wt[j] + sa[i]",
                      "S[i * N + j] = S[i * N + j] * wt[i] + sa[i]", 1),
    "checkpoint_one_token_late": ("if (ckpt && t % ORACLE_CHUNK == 0)",
                                  "if (ckpt && t % ORACLE_CHUNK == 1)", 1),
    "sequence_checkpoint_base_ignored": ("s[q].ckpt = seq_ckpt ? seq_ckpt[q] : 0;",
                                         "s[q].ckpt = 0;", 1),
    # backward
    "dS_missing_a_term": ("dS[i * N + j] = dS[i * N + j] * wt[j] + dsa[i] * at[j];",
                          "dS[i * N + j] = dS[i * N + j] * wt[j];", 1),
    "dw_uses_updated_state": ("acc_w += dS[i * N + j] * Sp[i * N + j];",
                              "acc_w += dS[i * N + j] * Sn[i * N + j];", 1),
    "dr_uses_previous_state": ("for (int i = 0; i < N; ++i) acc += Sn[i * N + j] * dy[o + i];",
                               "for (int i = 0; i < N; ++i) acc += Sp[i * N + j] * dy[o + i];", 1),
    "da_uses_dS_row_sum": ("acc_a += dsa[i] * Sp[i * N + j];",
                           "acc_a += dS[i * N + j] * Sp[i * N + j];", 1),
    "db_uses_v": ("acc_b += dS[i * N + j] * sa[i];",
                  "acc_b += dS[i * N + j] * vt[i];", 1),
}


def _all_pins_pass():
    failed = []
    for name, (fn, tol) in P.PINS.items():
        try:
            err = fn()
        except Exception as e:  # a crash of a pin counts as a detection
            failed.append((name, repr(e)))
            continue
        if not err <= tol:
            failed.append((name, err))
    return failed


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_mutation_is_caught(mutation, tmp_path):
    old, new, count = MUTATIONS[mutation]
    src = open(O.SRC).read()
    assert src.count(old) == count, f"mutation site not found exactly {count}x: {old!r}"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mut.c"
    so_path = tmp_path / "libmut.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    str(c_path), "-o", str(so_path)], check=True)
    with O.use_library(str(so_path)):
        failed = _all_pins_pass()
    assert failed, f"no pin detects mutation {mutation}"


def test_unmutated_oracle_passes_all_pins():
    assert _all_pins_pass() == []


# Slips in the fused decode epilogue (oracle.decode_step_fused, fp64 numpy):
# each is a full restatement of the epilogue with one mistake, checked
# against the p13 pins.
def _epilogue(mut):
    import numpy as np

    def f(r, w, k, v, a, b, s_in, g, ln_w, ln_b, r_k, eps):
        y, s_out = O.decode_step(r, w, k, v, a, b, s_in)
        y = np.asarray(y, dtype=np.float64)
        n = y.shape[-1]
        mean = y.mean(axis=-1, keepdims=True)
        var = ((y - mean) ** 2).sum(axis=-1, keepdims=True) / (n - 1 if mut == "sample_variance" else n)
        den = np.sqrt(var) + eps if mut == "eps_outside_sqrt" else np.sqrt(var + eps)
        yn = (y - mean) / den * ln_w[None] + ln_b[None]
        rk = {"bonus_without_r_k": np.ones_like(r_k), "r_k_of_other_head": r_k[::-1]}.get(mut, r_k)
        bonus = (r * k * rk[None]).sum(axis=-1, keepdims=True)
        if mut == "gate_before_bonus":
            return yn * g + bonus * v, y, s_out
        if mut == "bias_after_gate":
            return (yn - ln_b[None] + bonus * v) * g + ln_b[None], y, s_out
        if mut == "bonus_scales_r":
            return (yn + bonus * r) * g, y, s_out
        return (yn + bonus * v) * g, y, s_out
    return f


EPILOGUE_SLIPS = ["sample_variance", "eps_outside_sqrt", "bonus_without_r_k", "r_k_of_other_head",
                  "gate_before_bonus", "bias_after_gate", "bonus_scales_r"]


@pytest.mark.parametrize("mutation", EPILOGUE_SLIPS)
def test_epilogue_slip_is_caught(mutation, monkeypatch):
    monkeypatch.setattr(O, "decode_step_fused", _epilogue(mutation))
    failed = [n for n, (fn, tol) in P.PINS.items() if n.startswith("p13") and not fn() <= tol]
    assert failed, f"no pin detects epilogue slip {mutation}"


def test_epilogue_restatement_passes_pins(monkeypatch):
    monkeypatch.setattr(O, "decode_step_fused", _epilogue("none"))
    assert [n for n, (fn, tol) in P.PINS.items() if n.startswith("p13") and not fn() <= tol] == []


def _gdn(mut):
    """A restatement of the GDN remap with one planted slip."""
    def step(q, k, v, g, beta, s_in):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
        B, Hk, N = q.shape
        H = v.shape[1]
        kh = np.arange(H) // (H // Hk)
        qn = q if mut == "r_unnormalised" else q / np.linalg.norm(q, axis=-1, keepdims=True)
        kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
        kraw = k[:, kh] if mut == "kwrite_unnormalised" else kn[:, kh]
        r, kk = qn[:, kh], kn[:, kh]
        w = np.broadcast_to(np.exp(g)[..., None], (B, H, N))
        bt = beta[..., None]
        a = kk if mut == "a_sign" else -kk
        b = kk * (1.0 if mut == "b_no_decay" else np.exp(g)[..., None]) * (1.0 if mut == "b_no_beta" else bt)
        y, s_out = O.decode_step(r, w, bt * kraw, v, a, b, s_in)
        scale = 1.0 / N if mut == "scale_over_n" else 1.0 / np.sqrt(N)
        return np.asarray(y) * scale, s_out
    return step


GDN_SLIPS = ["a_sign", "b_no_beta", "b_no_decay", "scale_over_n", "kwrite_unnormalised",
             "r_unnormalised"]


@pytest.mark.parametrize("mutation", GDN_SLIPS)
def test_gdn_slip_is_caught(mutation, monkeypatch):
    monkeypatch.setattr(O, "gdn_decode_step", _gdn(mutation))
    failed = [n for n, (fn, tol) in P.PINS.items() if n.startswith("p15") and not fn() <= tol]
    assert failed, f"no pin detects GDN slip {mutation}"


def test_gdn_restatement_passes_pins(monkeypatch):
    monkeypatch.setattr(O, "gdn_decode_step", _gdn("none"))
    assert [n for n, (fn, tol) in P.PINS.items() if n.startswith("p15") and not fn() <= tol] == []


def _gdn_backward(mut):
    """A restatement of the GDN backward's chain rule with one planted slip."""
    def bwd(q, k, v, g, beta, s0=None, dout=None, ds_out=None):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
        B, T, Hk, N = q.shape
        H = v.shape[2]
        grp = H // Hk
        kh = np.arange(H) // grp
        qd = np.linalg.norm(q, axis=-1, keepdims=True)
        kd = np.linalg.norm(k, axis=-1, keepdims=True)
        qn, kn = q / qd, k / kd
        r, kk = qn[:, :, kh], kn[:, :, kh]
        dec, bt = np.exp(g)[..., None], beta[..., None]
        w = np.broadcast_to(dec, (B, T, H, N))
        gr = O.backward(r, w, bt * kk, v, -kk, kk * dec * bt, s0=s0,
                        dy=None if dout is None else dout / np.sqrt(N), ds_out=ds_out)
        dkk = bt * gr["dk"] + (gr["da"] if mut == "da_sign" else -gr["da"]) + bt * dec * gr["db"]
        dg = (1.0 if mut == "dg_no_decay" else np.exp(g)) * (
            np.sum(gr["dw"], axis=-1) + (0.0 if mut == "dg_no_b_term" else beta * np.sum(gr["db"] * kk, axis=-1)))
        dbeta = np.sum(gr["dk"] * kk, axis=-1) + (0.0 if mut == "dbeta_no_b_term" else np.exp(g) * np.sum(gr["db"] * kk, axis=-1))
        if mut == "no_group_sum":
            dqn, dkn = gr["dr"][:, :, ::grp], dkk[:, :, ::grp]
        else:
            dqn = gr["dr"].reshape(B, T, Hk, grp, N).sum(axis=3)
            dkn = dkk.reshape(B, T, Hk, grp, N).sum(axis=3)
        def through(xn, xd, dxn):
            if mut == "norm_no_projection":
                return dxn / xd
            return (dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)) / xd
        return {"dq": through(qn, qd, dqn), "dk": through(kn, kd, dkn), "dv": gr["dv"],
                "dg": dg, "dbeta": dbeta, "ds0": gr["ds0"]}
    return bwd


GDN_BACKWARD_SLIPS = ["da_sign", "dg_no_decay", "dg_no_b_term", "dbeta_no_b_term", "no_group_sum",
                      "norm_no_projection"]


@pytest.mark.parametrize("mutation", GDN_BACKWARD_SLIPS)
def test_gdn_backward_slip_is_caught(mutation, monkeypatch):
    monkeypatch.setattr(O, "gdn_backward", _gdn_backward(mutation))
    failed = [n for n, (fn, tol) in P.PINS.items() if n.startswith("p17") and not fn() <= tol]
    assert failed, f"no pin detects GDN backward slip {mutation}"


def test_gdn_backward_restatement_passes_pins(monkeypatch):
    monkeypatch.setattr(O, "gdn_backward", _gdn_backward("none"))
    assert [n for n, (fn, tol) in P.PINS.items() if n.startswith("p17") and not fn() <= tol] == []
