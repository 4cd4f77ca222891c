"""Pins of the fp64 oracle to things other than itself.

Every check below computes its expected value by a different route than the
oracle's token loop: closed forms of special cases, dense matrix products,
the textbook gated delta rule, invariants (state carry, packing, permutation,
linearity), exact gradient identities and central finite differences.
test_oracle_mutations.py shows that a plausible slip in the oracle trips at
least one of them.
"""
import numpy as np
import pytest

from oracle import oracle as O
from linear_recurrent_lm_amd import synth


def rand_inputs(B, T, H, N, seed, s0_std=0.0):
    inp = synth.make_inputs(B, T, H, N, seed=seed, dtype="f32", s0_std=s0_std)
    return [x.astype(np.float64) for x in inp.streams()], (
        None if inp.s0 is None else inp.s0.astype(np.float64))


def rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------- closed forms

def pin_p1(seed=1, B=2, T=37, H=2, N=16):
    """a = b = 0, w = 1: S_t = S_0 + sum_{s<=t} v_s k_s^T, y_t = S_t r_t."""
    (r, w, k, v, a, b), s0 = rand_inputs(B, T, H, N, seed, s0_std=0.3)
    w = np.ones_like(w); a = np.zeros_like(a); b = np.zeros_like(b)
    out = O.forward(r, w, k, v, a, b, s0=s0)
    outer = np.einsum("bthi,bthj->bthij", v, k)
    St = s0[:, None] + np.cumsum(outer, axis=1)          # [B,T,H,N,N]
    y_ref = np.einsum("bthij,bthj->bthi", St, r)
    return max(rel(out["y"], y_ref), rel(out["s_out"], St[:, -1]))


def pin_p2(seed=2, B=2, T=23, H=2, N=16):
    """a = b = 0, w = 0: S_t = v_t k_t^T whatever S_0; y_t = v_t (k_t . r_t)."""
    (r, w, k, v, a, b), s0 = rand_inputs(B, T, H, N, seed, s0_std=1.0)
    w = np.zeros_like(w); a = np.zeros_like(a); b = np.zeros_like(b)
    out = O.forward(r, w, k, v, a, b, s0=s0)
    y_ref = v * np.sum(k * r, axis=-1, keepdims=True)
    S_ref = np.einsum("bhi,bhj->bhij", v[:, -1], k[:, -1])
    return max(rel(out["y"], y_ref), rel(out["s_out"], S_ref))


def pin_p3(seed=3, T=29, N=12):
    """a = b = 0, general w: each S[i,j] is an independent scalar recurrence,
    S_T[i,j] = S_0[i,j] prod_t w_t[j] + sum_s v_s[i] k_s[j] prod_{u>s} w_u[j]."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, 1, N, seed, s0_std=0.5)
    a = np.zeros_like(a); b = np.zeros_like(b)
    out = O.forward(r, w, k, v, a, b, s0=s0)
    W = w[0, :, 0]                       # [T, N]
    S_ref = s0[0, 0] * np.prod(W, axis=0)[None, :]
    for s in range(T):
        tail = np.prod(W[s + 1:], axis=0) if s + 1 < T else np.ones(N)
        S_ref = S_ref + np.outer(v[0, s, 0], k[0, s, 0]) * tail[None, :]
    return rel(out["s_out"][0, 0], S_ref)


def pin_p4(seed=4, N=10):
    """T <= 4 brute force with dense transition matrices G_t = diag(w_t) +
    a_t b_t^T: S_t = S_0 G_1..G_t + sum_{s<=t} v_s k_s^T G_{s+1}..G_t."""
    worst = 0.0
    for T in (1, 2, 3, 4):
        (r, w, k, v, a, b), s0 = rand_inputs(1, T, 1, N, seed + T, s0_std=0.7)
        out = O.forward(r, w, k, v, a, b, s0=s0)
        G = [np.diag(w[0, t, 0]) + np.outer(a[0, t, 0], b[0, t, 0]) for t in range(T)]
        for t in range(T):
            St = s0[0, 0].copy()
            for u in range(t + 1):
                St = St @ G[u]
            for s in range(t + 1):
                P = np.outer(v[0, s, 0], k[0, s, 0])
                for u in range(s + 1, t + 1):
                    P = P @ G[u]
                St = St + P
            worst = max(worst, rel(out["y"][0, t, 0], St @ r[0, t, 0]))
        worst = max(worst, rel(out["s_out"][0, 0], St))
    return worst


def pin_p5(seed=5, T=40, N=16):
    """Gated delta rule special case: w = alpha*1, a = -kh, b = alpha*beta*kh,
    k = beta*kh, r = qh reproduces S_t = alpha S_{t-1}(I - beta kh kh^T) +
    beta v kh^T and o_t = S_t qh (the GDN-to-RWKV-7 remap on the rwkv-lab page)."""
    rng = np.random.default_rng(seed)
    kh = rng.standard_normal((T, N)); kh /= np.linalg.norm(kh, axis=1, keepdims=True)
    qh = rng.standard_normal((T, N)); qh /= np.linalg.norm(qh, axis=1, keepdims=True)
    v = rng.standard_normal((T, N))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.1, 1.0, T)
    s0 = rng.standard_normal((N, N)) * 0.3
    S = s0.copy(); o_ref = np.zeros((T, N))
    for t in range(T):
        S = alpha[t] * S @ (np.eye(N) - beta[t] * np.outer(kh[t], kh[t])) \
            + beta[t] * np.outer(v[t], kh[t])
        o_ref[t] = S @ qh[t]
    sh = lambda x: x.reshape(1, T, 1, N)
    out = O.forward(sh(qh), sh(np.repeat(alpha[:, None], N, 1)),
                    sh(beta[:, None] * kh), sh(v), sh(-kh),
                    sh((alpha * beta)[:, None] * kh), s0=s0.reshape(1, 1, N, N))
    e = max(rel(out["y"][0, :, 0], o_ref), rel(out["s_out"][0, 0], S))
    # alpha = beta = 1: the delta rule writes v exactly, so reading with r = kh returns v.
    out1 = O.forward(sh(kh), sh(np.ones((T, N))), sh(kh), sh(v), sh(-kh), sh(kh),
                     s0=s0.reshape(1, 1, N, N))
    return max(e, rel(out1["y"][0, :, 0], v))


# ---------------------------------------------------------------- invariants

def pin_p6_forward(seed=6, T=53, H=2, N=16, splits=(1, 16, 17, 30, 52)):
    """Split-sequence state carry: run(x[:T]) == run(x[T1:], s0=run(x[:T1]).S_T),
    and every checkpoint equals the state after 16c tokens."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, H, N, seed, s0_std=0.2)
    full = O.forward(r, w, k, v, a, b, s0=s0, checkpoints=True)
    worst = 0.0
    for T1 in splits:
        p1 = O.forward(*[x[:, :T1] for x in (r, w, k, v, a, b)], s0=s0)
        p2 = O.forward(*[x[:, T1:] for x in (r, w, k, v, a, b)], s0=p1["s_out"])
        y = np.concatenate([p1["y"], p2["y"]], axis=1)
        worst = max(worst, rel(y, full["y"]), rel(p2["s_out"], full["s_out"]))
    nc = -(-T // 16)
    assert full["ckpt"].shape == (nc, H, N, N)
    worst = max(worst, rel(full["ckpt"][0], s0[0]))
    for c in range(1, nc):
        pc = O.forward(*[x[:, :16 * c] for x in (r, w, k, v, a, b)], s0=s0)
        worst = max(worst, rel(full["ckpt"][c], pc["s_out"][0]))
    return worst


def pin_p6_backward(seed=7, T=41, H=1, N=12, T1=19):
    """Carry of the adjoint: the backward of the second half returns, as ds0,
    the ds_out that the first half's backward must receive."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, H, N, seed, s0_std=0.2)
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal(r.shape)
    dso = rng.standard_normal((1, H, N, N))
    full = O.backward(r, w, k, v, a, b, s0=s0, dy=dy, ds_out=dso)
    first = O.forward(*[x[:, :T1] for x in (r, w, k, v, a, b)], s0=s0)
    g2 = O.backward(*[x[:, T1:] for x in (r, w, k, v, a, b)], s0=first["s_out"],
                    dy=dy[:, T1:], ds_out=dso)
    g1 = O.backward(*[x[:, :T1] for x in (r, w, k, v, a, b)], s0=s0,
                    dy=dy[:, :T1], ds_out=g2["ds0"])
    worst = rel(g1["ds0"], full["ds0"])
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        worst = max(worst, rel(np.concatenate([g1[n], g2[n]], axis=1), full[n]))
    return worst


def pin_p7(seed=8, T=9, H=3, N=16):
    """T decode steps equal one forward over T tokens."""
    (r, w, k, v, a, b), s0 = rand_inputs(2, T, H, N, seed, s0_std=0.1)
    full = O.forward(r, w, k, v, a, b, s0=s0)
    S = s0.copy(); worst = 0.0
    for t in range(T):
        y, S = O.decode_step(*[x[:, t] for x in (r, w, k, v, a, b)], S)
        worst = max(worst, rel(y, full["y"][:, t]))
    return max(worst, rel(S, full["s_out"]))


def pin_p8(seed=9, H=2, N=16):
    """Packed streams with resets == sequences run one by one == right-padded
    rows with lengths; NaN in padding never reaches any output."""
    lengths = np.array([5, 16, 33, 1, 20, 17, 8], dtype=np.int32)
    flat, s0 = synth.make_segment_inputs(lengths, H, N, seed=seed, dtype="f32",
                                         s0_std=0.2, with_dy=True)
    names = ("r", "w", "k", "v", "a", "b")
    T_pad, st_p, ln = synth.packed_layout(lengths, 3)
    packed = synth.scatter_segments(flat, lengths, st_p, 3, T_pad, dtype="f32")
    T_r = int(lengths.max()) + 3
    st_r, _ = synth.padded_layout(lengths, T_r)
    padded = synth.scatter_segments(flat, lengths, st_r, len(lengths), T_r, dtype="f32")
    worst = 0.0
    outs = []
    for lay in (packed, padded):
        f = O.forward(*[getattr(lay, n) for n in names], s0=s0, seq_start=lay.seq_start,
                      seq_len=lay.seq_len, checkpoints=True)
        g = O.backward(*[getattr(lay, n) for n in names], s0=s0, dy=lay.dy,
                       seq_start=lay.seq_start, seq_len=lay.seq_len)
        for arr in list(f.values()) + list(g.values()):
            assert np.all(np.isfinite(arr))
        outs.append((lay, f, g))
    off = 0
    for i, L in enumerate(lengths):
        sep = [flat[n][off:off + L][None, :] for n in names]
        f1 = O.forward(*sep, s0=s0[i:i + 1], checkpoints=True)
        g1 = O.backward(*sep, s0=s0[i:i + 1], dy=flat["dy"][off:off + L][None, :])
        for lay, f, g in outs:
            st = int(lay.seq_start[i]); Bt = lay.r.shape[1]
            bb, t0 = divmod(st, Bt)
            worst = max(worst, rel(f["y"][bb, t0:t0 + L], f1["y"][0]))
            worst = max(worst, rel(f["s_out"][i], f1["s_out"][0]))
            base = int(f["ckpt_base"][i])
            nc = -(-L // 16)
            worst = max(worst, rel(f["ckpt"][base:base + nc], f1["ckpt"]))
            for n in ("dr", "dw", "dk", "dv", "da", "db"):
                worst = max(worst, rel(g[n][bb, t0:t0 + L], g1[n][0]))
            worst = max(worst, rel(g["ds0"][i], g1["ds0"][0]))
        off += L
    return worst


def pin_p9(seed=10, T=21, N=12):
    """Permuting value rows permutes S's rows and y's channels; permuting key
    columns (r, w, k, a, b and S_0's columns) permutes S's columns, y unchanged."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, 1, N, seed, s0_std=0.4)
    base = O.forward(r, w, k, v, a, b, s0=s0)
    pv = np.random.default_rng(seed).permutation(N)
    pk = np.random.default_rng(seed + 1).permutation(N)
    o1 = O.forward(r, w, k, v[..., pv], a, b, s0=s0[:, :, pv, :])
    o2 = O.forward(r[..., pk], w[..., pk], k[..., pk], v, a[..., pk], b[..., pk],
                   s0=s0[:, :, :, pk])
    return max(rel(o1["y"], base["y"][..., pv]), rel(o1["s_out"], base["s_out"][:, :, pv, :]),
               rel(o2["y"], base["y"]), rel(o2["s_out"], base["s_out"][:, :, :, pk]))


def pin_p10(seed=11, T=19, N=12):
    """(y, S_T) is linear in (v, S_0) jointly and in (k, S_0) jointly; y_t is
    linear in r_t."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, 1, N, seed, s0_std=0.4)
    (_, _, k2, v2, _, _), s02 = rand_inputs(1, T, 1, N, seed + 100, s0_std=0.4)
    r2 = rand_inputs(1, T, 1, N, seed + 200)[0][0]
    f = lambda **kw: O.forward(**{**dict(r=r, w=w, k=k, v=v, a=a, b=b, s0=s0), **kw})
    base = f()
    c1, c2 = 0.7, -1.3
    worst = 0.0
    lin = f(v=c1 * v + c2 * v2, s0=c1 * s0 + c2 * s02)
    o2 = f(v=v2, s0=s02)
    worst = max(worst, rel(lin["y"], c1 * base["y"] + c2 * o2["y"]),
                rel(lin["s_out"], c1 * base["s_out"] + c2 * o2["s_out"]))
    lin = f(k=c1 * k + c2 * k2, s0=c1 * s0 + c2 * s02)
    o2 = f(k=k2, s0=s02)
    worst = max(worst, rel(lin["y"], c1 * base["y"] + c2 * o2["y"]),
                rel(lin["s_out"], c1 * base["s_out"] + c2 * o2["s_out"]))
    lin = f(r=c1 * r + c2 * r2)
    o2 = f(r=r2)
    return max(worst, rel(lin["y"], c1 * base["y"] + c2 * o2["y"]))


def pin_p11(seed=12, B=2, T=27, H=2, N=16):
    """Exact gradient identities for L = sum <dy,y> + <ds_out,S_T>:
    <dr_t,r_t> = <dy_t,y_t>; <dv_t,v_t> = <dk_t,k_t>; <da_t,a_t> = <db_t,b_t>;
    sum_t <dv_t,v_t> + <ds0,S_0> = L (L is degree-1 homogeneous in (v, S_0))."""
    (r, w, k, v, a, b), s0 = rand_inputs(B, T, H, N, seed, s0_std=0.3)
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal(r.shape); dso = rng.standard_normal(s0.shape)
    f = O.forward(r, w, k, v, a, b, s0=s0)
    g = O.backward(r, w, k, v, a, b, s0=s0, dy=dy, ds_out=dso)
    dot = lambda x, y: np.sum(x * y, axis=-1)
    worst = 0.0
    for lhs, rhs in ((dot(g["dr"], r), dot(dy, f["y"])),
                     (dot(g["dv"], v), dot(g["dk"], k)),
                     (dot(g["da"], a), dot(g["db"], b))):
        worst = max(worst, rel(lhs, rhs))
    L = np.sum(dy * f["y"]) + np.sum(dso * f["s_out"])
    euler = np.sum(g["dv"] * v) + np.sum(g["ds0"] * s0)
    return max(worst, abs(L - euler) / abs(L))


def pin_p12(seed=13, T=6, N=5, eps=1e-6):
    """Central finite differences of L w.r.t. every input element and S_0."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, T, 1, N, seed, s0_std=0.5)
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal(r.shape); dso = rng.standard_normal(s0.shape)
    args = dict(r=r, w=w, k=k, v=v, a=a, b=b, s0=s0)

    def loss(**kw):
        o = O.forward(**{**args, **kw})
        return np.sum(dy * o["y"]) + np.sum(dso * o["s_out"])

    g = O.backward(r, w, k, v, a, b, s0=s0, dy=dy, ds_out=dso)
    worst = 0.0
    for name, gname in (("r", "dr"), ("w", "dw"), ("k", "dk"), ("v", "dv"),
                        ("a", "da"), ("b", "db"), ("s0", "ds0")):
        x = args[name]; fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = eps * max(1.0, abs(x[idx]))
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
        worst = max(worst, rel(g[gname], fd))
    return worst


# ------------------------------------------- fused decode epilogue (reading)

def _fused_inputs(seed, B=3, H=2, N=16):
    (r, w, k, v, a, b), s0 = rand_inputs(B, 1, H, N, seed, s0_std=0.3)
    r, w, k, v, a, b = (x[:, 0] for x in (r, w, k, v, a, b))
    rng = np.random.default_rng(seed)
    g = rng.normal(size=r.shape)
    ln_w = rng.normal(size=(H, N)); ln_b = rng.normal(size=(H, N)); r_k = rng.normal(size=(H, N))
    return [r, w, k, v, a, b], s0, g, ln_w, ln_b, r_k


def _y_equals_v(r, w, k, v, a, b, s0):
    """Inputs whose decode output is exactly v: zero state, a = b = 0 and
    r = k / |k|^2 give y = v (k . r) = v."""
    k = k.copy()
    r = k / np.sum(k * k, axis=-1, keepdims=True)
    return [r, w, k, v, np.zeros_like(a), np.zeros_like(b)], np.zeros_like(s0)


def pin_p13_normalised(seed=31):
    """eps = 0, unit affine, no bonus, g = 1: each head's output has mean 0
    and population variance 1."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    out, _, _ = O.decode_step_fused(*st, s0, np.ones_like(g), np.ones_like(ln_w),
                                    np.zeros_like(ln_b), np.zeros_like(r_k), 0.0)
    return max(float(np.max(np.abs(out.mean(axis=-1)))),
               float(np.max(np.abs((out ** 2).mean(axis=-1) - 1.0))))


def pin_p13_affine_invariance(seed=32):
    """eps = 0, no bonus: replacing y by alpha y + beta (alpha > 0) leaves the
    output unchanged (y = v by construction)."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    st, s0 = _y_equals_v(*st, s0)
    z = np.zeros_like(r_k)
    out1, _, _ = O.decode_step_fused(*st, s0, g, ln_w, ln_b, z, 0.0)
    st2 = list(st); st2[3] = 2.5 * st[3] - 0.7
    out2, _, _ = O.decode_step_fused(*st2, s0, g, ln_w, ln_b, z, 0.0)
    return rel(out2, out1)


def pin_p13_eps_closed_form(seed=33, eps=0.37):
    """y = alternating +-1 per head (mean 0, variance 1), unit affine, no bonus,
    g = 1: out = y / sqrt(1 + eps)."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    st, s0 = _y_equals_v(*st, s0)
    N = st[3].shape[-1]
    st[3] = np.broadcast_to(np.where(np.arange(N) % 2 == 0, 1.0, -1.0), st[3].shape).copy()
    out, _, _ = O.decode_step_fused(*st, s0, np.ones_like(g), np.ones_like(ln_w),
                                    np.zeros_like(ln_b), np.zeros_like(r_k), eps)
    return rel(out, st[3] / np.sqrt(1.0 + eps))


def pin_p13_bonus_dot(seed=34):
    """Zero affine, r_k = 1, g = 1: out = (r . k) v, the dot product by numpy."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    out, _, _ = O.decode_step_fused(*st, s0, np.ones_like(g), np.zeros_like(ln_w),
                                    np.zeros_like(ln_b), np.ones_like(r_k), 1e-5)
    r, k, v = st[0], st[2], st[3]
    dots = np.array([[np.dot(r[bb, h], k[bb, h]) for h in range(r.shape[1])] for bb in range(r.shape[0])])
    return rel(out, dots[..., None] * v)


def pin_p13_bonus_locality(seed=37):
    """Zero affine, g = 1, r_k nonzero on head 0 only: the other heads output
    zero, and head 0's output is homogeneous of degree 1 in r_k."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    r_k[1:] = 0.0
    z, one = np.zeros_like(ln_w), np.ones_like(g)
    out1, _, _ = O.decode_step_fused(*st, s0, one, z, z, r_k, 1e-5)
    out2, _, _ = O.decode_step_fused(*st, s0, one, z, z, 2.0 * r_k, 1e-5)
    return max(float(np.max(np.abs(out1[:, 1:]))), rel(out2, 2.0 * out1))


def pin_p13_gate_and_bias(seed=35):
    """The gate scales the whole output elementwise, and a bias shift delta
    moves the output by delta * g."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    out_g, _, _ = O.decode_step_fused(*st, s0, g, ln_w, ln_b, r_k, 1e-3)
    out_1, _, _ = O.decode_step_fused(*st, s0, np.ones_like(g), ln_w, ln_b, r_k, 1e-3)
    delta = np.linspace(-1.0, 1.0, ln_b.size).reshape(ln_b.shape)
    out_d, _, _ = O.decode_step_fused(*st, s0, g, ln_w, ln_b + delta, r_k, 1e-3)
    return max(rel(out_g, out_1 * g), rel(out_d - out_g, delta[None] * g))


def pin_p13_state_unchanged(seed=36):
    """y and the new state are the plain decode step's."""
    st, s0, g, ln_w, ln_b, r_k = _fused_inputs(seed)
    _, y, s1 = O.decode_step_fused(*st, s0, g, ln_w, ln_b, r_k, 1e-5)
    y_ref, s_ref = O.decode_step(*st, s0)
    return max(rel(y, y_ref), rel(s1, s_ref))



# P15: the GDN remap (rwkv-lab, "Highlight result -- GDN in RWKV-7").
def _gdn_inputs(seed, B=2, Hk=2, H=4, N=128):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, Hk, N))
    k = rng.standard_normal((B, Hk, N))
    v = rng.standard_normal((B, H, N))
    g = -rng.uniform(0.01, 1.0, (B, H))
    beta = rng.uniform(0.05, 1.0, (B, H))
    s = 0.1 * rng.standard_normal((B, H, N, N))
    return q, k, v, g, beta, s


def _gdn_textbook(q, k, v, g, beta, s):
    """The gated delta rule written as matrices, per (b, value head):
    S' = exp(g) S (I - beta k^ k^T) + beta v k^T,  o = S' q^ / sqrt(N)."""
    B, Hk, N = q.shape
    H = v.shape[1]
    out = np.empty((B, H, N))
    s1 = np.empty_like(s)
    for b in range(B):
        for h in range(H):
            kh = h // (H // Hk)
            qh = q[b, kh] / np.linalg.norm(q[b, kh])
            kk = k[b, kh] / np.linalg.norm(k[b, kh])
            S = np.exp(g[b, h]) * s[b, h] @ (np.eye(N) - beta[b, h] * np.outer(kk, kk)) \
                + beta[b, h] * np.outer(v[b, h], kk)
            s1[b, h] = S
            out[b, h] = S @ qh / np.sqrt(N)
    return out, s1


def pin_p15_gated_delta_rule(seed=37):
    """The remapped WKV-7 step equals the textbook gated delta rule (N = 128
    and N = 64, two value heads per key head)."""
    err = 0.0
    for N in (128, 64):
        inp = _gdn_inputs(seed, N=N)
        o1, s1 = O.gdn_decode_step(*inp)
        o2, s2 = _gdn_textbook(*inp)
        err = max(err, rel(o1, o2), rel(s1, s2))
    return err


def pin_p15_delta_writes_v(seed=38):
    """With no decay and beta = 1 the delta rule overwrites the value stored
    at key k^: the new state maps k^ to v exactly."""
    q, k, v, g, beta, s = _gdn_inputs(seed)
    _, s1 = O.gdn_decode_step(q, k, v, np.zeros_like(g), np.ones_like(beta), s)
    err = 0.0
    for b in range(2):
        for h in range(4):
            kk = k[b, h // 2] / np.linalg.norm(k[b, h // 2])
            err = max(err, rel(s1[b, h] @ kk, v[b, h]))
    return err


def pin_p15_beta_zero(seed=39):
    """beta = 0 only decays the state: S' = exp(g) S, o = exp(g) S q^ / sqrt(N)."""
    q, k, v, g, beta, s = _gdn_inputs(seed)
    o1, s1 = O.gdn_decode_step(q, k, v, g, np.zeros_like(beta), s)
    s_want = np.exp(g)[..., None, None] * s
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    o_want = np.einsum("bhij,bhj->bhi", s_want, qn[:, [0, 0, 1, 1]]) / np.sqrt(128)
    return max(rel(s1, s_want), rel(o1, o_want))


def pin_p15_norm_invariance(seed=40):
    """q and k enter only through their directions."""
    q, k, v, g, beta, s = _gdn_inputs(seed)
    o1, s1 = O.gdn_decode_step(q, k, v, g, beta, s)
    o2, s2 = O.gdn_decode_step(3.7 * q, 0.21 * k, v, g, beta, s)
    return max(rel(o2, o1), rel(s2, s1))


def pin_p16_gdn_forward_textbook(seed=41):
    """A sequence of GDN tokens equals the textbook gated delta rule applied
    token by token (N = 128, two value heads per key head, random s0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hk, H, N = 2, 6, 2, 4, 128
    q = rng.standard_normal((B, T, Hk, N))
    k = rng.standard_normal((B, T, Hk, N))
    v = rng.standard_normal((B, T, H, N))
    g = -rng.uniform(0.01, 1.0, (B, T, H))
    beta = rng.uniform(0.05, 1.0, (B, T, H))
    s = 0.1 * rng.standard_normal((B, H, N, N))
    out, s_out = O.gdn_forward(q, k, v, g, beta, s)
    err = 0.0
    for t in range(T):
        o_t, s = _gdn_textbook(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], s)
        err = max(err, rel(out[:, t], o_t))
    return max(err, rel(s_out, s))


def pin_p16_gdn_forward_zero_state(seed=42):
    """Without s0 the sequence starts from the zero state: the first token's
    output is beta_0 <k^_0, q^_0> v_0 / sqrt(N)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hk, H, N = 1, 3, 1, 2, 64
    q = rng.standard_normal((B, T, Hk, N))
    k = rng.standard_normal((B, T, Hk, N))
    v = rng.standard_normal((B, T, H, N))
    g = -rng.uniform(0.01, 1.0, (B, T, H))
    beta = rng.uniform(0.05, 1.0, (B, T, H))
    out, _ = O.gdn_forward(q, k, v, g, beta)
    qn = q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    kn = k[0, 0, 0] / np.linalg.norm(k[0, 0, 0])
    want = beta[0, 0, :, None] * np.dot(kn, qn) * v[0, 0] / np.sqrt(N)
    return rel(out[0, 0], want)

def pin_p16_gdn_zero_rows(seed=43):
    """A token whose k is all zero only decays the state (S_t = e^g S_{t-1}),
    and a token whose q is all zero outputs exactly zero: the normalisation
    x / max(||x||, 1e-12) sends a zero row to zero instead of 0/0. Both are
    checked in the middle of a sequence, with every later token against the
    textbook rule from the decayed state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, Hk, H, N = 2, 7, 2, 4, 128
    q = rng.standard_normal((B, T, Hk, N))
    k = rng.standard_normal((B, T, Hk, N))
    v = rng.standard_normal((B, T, H, N))
    g = -rng.uniform(0.01, 1.0, (B, T, H))
    beta = rng.uniform(0.05, 1.0, (B, T, H))
    s = 0.1 * rng.standard_normal((B, H, N, N))
    k[:, 3] = 0.0
    q[:, 5] = 0.0
    out, s_out = O.gdn_forward(q, k, v, g, beta, s)
    if not (np.all(np.isfinite(out)) and np.all(np.isfinite(s_out))):
        return np.inf
    err = float(np.max(np.abs(out[:, 5])))                 # zero q: zero output
    st = s
    for t in range(T):
        if t == 3:                                        # zero k: decay only
            st = np.exp(g[:, t])[..., None, None] * st
            qn = q[:, t] / np.linalg.norm(q[:, t], axis=-1, keepdims=True)
            o_t = np.einsum("bhij,bhj->bhi", st, qn[:, [0, 0, 1, 1]]) / np.sqrt(N)
        elif t == 5:
            _, st = _gdn_textbook(np.ones_like(q[:, t]), k[:, t], v[:, t], g[:, t], beta[:, t], st)
            o_t = np.zeros_like(out[:, t])
        else:
            o_t, st = _gdn_textbook(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], st)
        err = max(err, rel(out[:, t], o_t))
    return max(err, rel(s_out, st))


# P17: the GDN backward through the remap (oracle.gdn_backward).
def _gdn_seq(seed, B, T, Hk, H, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, T, Hk, N))
    k = rng.standard_normal((B, T, Hk, N))
    v = rng.standard_normal((B, T, H, N))
    g = -rng.uniform(0.01, 1.0, (B, T, H))
    beta = rng.uniform(0.05, 1.0, (B, T, H))
    s0 = 0.3 * rng.standard_normal((B, H, N, N))
    dout = rng.standard_normal((B, T, H, N))
    dso = rng.standard_normal((B, H, N, N))
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0), dout, dso


def pin_p17_gdn_finite_differences(seed=51, eps=1e-6):
    """Central finite differences of L = sum <dout, out> + <ds_out, S_T>
    through gdn_forward, w.r.t. every element of q, k, v, g, beta and S_0
    (two value heads over one key head, N = 6)."""
    args, dout, dso = _gdn_seq(seed, 1, 4, 1, 2, 6)

    def loss(**kw):
        out, s_out = O.gdn_forward(**{**args, **kw})
        return np.sum(dout * out) + np.sum(dso * s_out)

    gb = O.gdn_backward(**args, dout=dout, ds_out=dso)
    worst = 0.0
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"),
                        ("beta", "dbeta"), ("s0", "ds0")):
        x = args[name]; fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = eps * max(1.0, abs(x[idx]))
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
        worst = max(worst, rel(gb[gname], fd))
    return worst


def pin_p17_gdn_identities(seed=52):
    """At N = 128 (32 value heads' geometry scaled down to 4 over 2 key
    heads): <dq, q> = <dk, k> = 0 per token and key head (the output does
    not depend on the lengths of q and k); sum <dv, v> + <ds0, S_0> = L (out
    and S_T are linear in (v, S_0) jointly); with beta = 0 nothing is
    written, so dk = dv = 0 exactly."""
    args, dout, dso = _gdn_seq(seed, 2, 5, 2, 4, 128)
    out, s_out = O.gdn_forward(**args)
    gb = O.gdn_backward(**args, dout=dout, ds_out=dso)
    L = np.sum(dout * out) + np.sum(dso * s_out)
    scale = np.max(np.abs(gb["dq"])) * np.max(np.abs(args["q"])) * 128
    worst = float(np.max(np.abs(np.sum(gb["dq"] * args["q"], axis=-1)))) / scale
    scale = np.max(np.abs(gb["dk"])) * np.max(np.abs(args["k"])) * 128
    worst = max(worst, float(np.max(np.abs(np.sum(gb["dk"] * args["k"], axis=-1)))) / scale)
    euler = np.sum(gb["dv"] * args["v"]) + np.sum(gb["ds0"] * args["s0"])
    worst = max(worst, abs(L - euler) / abs(L))
    g0 = O.gdn_backward(**{**args, "beta": np.zeros_like(args["beta"])}, dout=dout, ds_out=dso)
    return max(worst, float(np.max(np.abs(g0["dk"]))), float(np.max(np.abs(g0["dv"]))))


PINS = {
    "p1_cumulative": (pin_p1, 1e-12),
    "p2_w0_last_outer": (pin_p2, 1e-12),
    "p3_scalar_recurrences": (pin_p3, 1e-12),
    "p4_bruteforce_products": (pin_p4, 1e-12),
    "p5_gated_delta_rule": (pin_p5, 1e-12),
    "p6_split_carry_forward": (pin_p6_forward, 1e-12),
    "p6_split_carry_backward": (pin_p6_backward, 1e-12),
    "p7_decode_equals_forward": (pin_p7, 1e-12),
    "p8_packed_padded_separate": (pin_p8, 1e-12),
    "p9_permutations": (pin_p9, 1e-12),
    "p10_linearity": (pin_p10, 1e-12),
    "p11_gradient_identities": (pin_p11, 1e-10),
    "p12_finite_differences": (pin_p12, 1e-6),
    "p13_fused_normalised": (pin_p13_normalised, 1e-12),
    "p13_fused_affine_invariance": (pin_p13_affine_invariance, 1e-12),
    "p13_fused_eps_closed_form": (pin_p13_eps_closed_form, 1e-12),
    "p13_fused_bonus_dot": (pin_p13_bonus_dot, 1e-12),
    "p13_fused_gate_and_bias": (pin_p13_gate_and_bias, 1e-12),
    "p13_fused_bonus_locality": (pin_p13_bonus_locality, 1e-12),
    "p13_fused_state_unchanged": (pin_p13_state_unchanged, 0.0),
    "p15_gdn_gated_delta_rule": (pin_p15_gated_delta_rule, 1e-12),
    "p15_gdn_delta_writes_v": (pin_p15_delta_writes_v, 1e-12),
    "p15_gdn_beta_zero": (pin_p15_beta_zero, 1e-12),
    "p15_gdn_norm_invariance": (pin_p15_norm_invariance, 1e-12),
    "p16_gdn_forward_textbook": (pin_p16_gdn_forward_textbook, 1e-12),
    "p16_gdn_forward_zero_state": (pin_p16_gdn_forward_zero_state, 1e-12),
    "p16_gdn_zero_rows": (pin_p16_gdn_zero_rows, 1e-12),
    "p17_gdn_backward_finite_differences": (pin_p17_gdn_finite_differences, 1e-6),
    "p17_gdn_backward_identities": (pin_p17_gdn_identities, 1e-12),
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_p2_initial_state_forgotten():
    """With w = 0 and a = b = 0 the initial state is wiped at the first token."""
    (r, w, k, v, a, b), s0 = rand_inputs(1, 4, 1, 8, 21, s0_std=5.0)
    w[:] = 0; a[:] = 0; b[:] = 0
    g = O.backward(r, w, k, v, a, b, s0=s0, dy=np.ones_like(r))
    assert np.all(g["ds0"] == 0)


def test_checkpoint_layout_dense():
    """Dense checkpoints: row b's chunk c at slot b*ceil(T/16)+c."""
    (r, w, k, v, a, b), s0 = rand_inputs(3, 33, 2, 8, 22, s0_std=0.2)
    out = O.forward(r, w, k, v, a, b, s0=s0, checkpoints=True)
    assert out["ckpt"].shape == (3 * 3, 2, 8, 8)
    for bb in range(3):
        assert np.array_equal(out["ckpt"][bb * 3], s0[bb])
