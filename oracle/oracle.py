"""Python front of the fp64 WKV-7 oracle (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. It loads `libwkv7_oracle.so`, built from
`wkv7_oracle.c` in this directory by `build()`, and shares nothing with the
GPU library. All inputs are upcast to fp64 (exact for fp32 and bf16 values).

Semantics follow the token-order definition written out in wkv7_oracle.c:
per (sequence, head) unit, S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T
+ v_t k_t^T and y_t = S_t r_t, with state checkpoints every 16 tokens and the
backward of L = sum <dy, y> + <ds_out, S_T>.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "wkv7_oracle.c")
LIB = os.path.join(HERE, "libwkv7_oracle.so")
CHUNK = 16

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: fp64, -O2, no fast-math, OpenMP."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _configure(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i = ctypes.c_int
    lib.wkv7o_forward.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                  i, ip, ip, ip, dp, dp, dp, dp, i, ip, i]
    lib.wkv7o_forward.restype = i
    lib.wkv7o_backward.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                   i, ip, ip, dp, dp, dp,
                                   dp, dp, dp, dp, dp, dp, dp, i, ip, i]
    lib.wkv7o_backward.restype = i
    lib.wkv7o_max_threads.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        _lib = _configure(ctypes.CDLL(LIB))
    return _lib


class use_library:
    """Context manager: route this module's calls through another build of
    the oracle (the mutation tests load deliberately broken copies)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _configure(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def max_threads() -> int:
    return int(_load().wkv7o_max_threads())


def _d(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x, t=ctypes.c_double):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(t))


def _segments(B, T, seq_start, seq_len):
    if seq_start is None:
        return 0, None, None, B
    st = np.ascontiguousarray(seq_start, dtype=np.int32)
    ln = np.ascontiguousarray(seq_len, dtype=np.int32)
    return len(st), st, ln, len(st)


def checkpoint_slots(T, seq_len=None, B=None):
    """Checkpoint slot bases and total: dense rows use ceil(T/16) slots each."""
    if seq_len is None:
        nc = -(-T // CHUNK)
        return np.arange(B, dtype=np.int32) * nc, B * nc
    n = (np.asarray(seq_len, dtype=np.int64) + CHUNK - 1) // CHUNK
    base = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int32) if len(n) else np.zeros(0, np.int32)
    return base, int(n.sum())


def forward(r, w, k, v, a, b, s0=None, *, seq_start=None, seq_len=None,
            checkpoints=False, units=None, threads=0):
    """Token-order fp64 forward.

    Streams are [B, T, H, N]. Returns dict with y [B,T,H,N] (zeros at tokens
    outside computed units), s_out [S,H,N,N] and, if requested, ckpt
    [slots,H,N,N]. `units` is an optional list of (sequence, head) pairs."""
    lib = _load()
    B, T, H, N = r.shape
    arrs = [_d(x) for x in (r, w, k, v, a, b)]
    nseq, st, ln, S = _segments(B, T, seq_start, seq_len)
    s0d = _d(s0)
    y = np.zeros((B, T, H, N), dtype=np.float64)
    s_out = np.zeros((S, H, N, N), dtype=np.float64)
    ckpt = None
    ck_base = None
    if checkpoints:
        ck_base, slots = checkpoint_slots(T, ln, B)
        ckpt = np.zeros((slots, H, N, N), dtype=np.float64)
    u = None if units is None else np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    rc = lib.wkv7o_forward(B, T, H, N, *[_p(x) for x in arrs], nseq,
                           _p(st, ctypes.c_int32), _p(ln, ctypes.c_int32),
                           _p(ck_base if nseq else None, ctypes.c_int32),
                           _p(s0d), _p(y), _p(s_out), _p(ckpt),
                           0 if u is None else len(u), _p(u, ctypes.c_int32), threads)
    if rc != 0:
        raise RuntimeError("oracle forward failed")
    out = {"y": y, "s_out": s_out}
    if checkpoints:
        out["ckpt"] = ckpt
        out["ckpt_base"] = ck_base
    return out


def backward(r, w, k, v, a, b, s0=None, dy=None, ds_out=None, *, seq_start=None,
             seq_len=None, units=None, threads=0):
    """fp64 reverse-mode gradients of L = sum <dy, y> + <ds_out, S_T>.
    Returns dict dr, dw, dk, dv, da, db ([B,T,H,N]) and ds0 ([S,H,N,N])."""
    lib = _load()
    B, T, H, N = r.shape
    arrs = [_d(x) for x in (r, w, k, v, a, b)]
    nseq, st, ln, S = _segments(B, T, seq_start, seq_len)
    grads = [np.zeros((B, T, H, N), dtype=np.float64) for _ in range(6)]
    ds0 = np.zeros((S, H, N, N), dtype=np.float64)
    u = None if units is None else np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    rc = lib.wkv7o_backward(B, T, H, N, *[_p(x) for x in arrs], nseq,
                            _p(st, ctypes.c_int32), _p(ln, ctypes.c_int32),
                            _p(_d(s0)), _p(_d(dy)), _p(_d(ds_out)),
                            *[_p(g) for g in grads], _p(ds0),
                            0 if u is None else len(u), _p(u, ctypes.c_int32), threads)
    if rc != 0:
        raise RuntimeError("oracle backward: out of memory for the state history")
    names = ("dr", "dw", "dk", "dv", "da", "db")
    out = dict(zip(names, grads))
    out["ds0"] = ds0
    return out


def decode_step(r, w, k, v, a, b, s_in):
    """One token per (sequence, head): streams [B, H, N], state [B, H, N, N].
    Returns (y [B,H,N], s_out [B,H,N,N])."""
    B, H, N = r.shape
    streams = [np.asarray(x).reshape(B, 1, H, N) for x in (r, w, k, v, a, b)]
    out = forward(*streams, s0=s_in)
    return out["y"].reshape(B, H, N), out["s_out"]


def decode_step_fused(r, w, k, v, a, b, s_in, g, ln_w, ln_b, r_k, eps):
    """One decode step followed by the per-head output epilogue that the
    rwkv-lab page ("RWKV community research additions") fuses into its
    one-token kernel: GroupNorm, the RWKV bonus and output gating. The
    rwkv-metal page ("What's inside") names ln_x a GroupNorm per head. The
    pages print no formula; the reading taken, per (sequence, head) h with
    population mean and variance over the head's N values of y:

        yn_i  = (y_i - mean(y)) / sqrt(var(y) + eps) * ln_w[h, i] + ln_b[h, i]
        out_i = (yn_i + (sum_j r_j k_j r_k[h, j]) * v_i) * g_i

    Streams and g [B, H, N]; ln_w, ln_b, r_k [H, N]; state [B, H, N, N].
    Returns (out, y, s_out), all fp64."""
    y, s_out = decode_step(r, w, k, v, a, b, s_in)
    y = np.asarray(y, dtype=np.float64)
    mean = y.mean(axis=-1, keepdims=True)
    var = ((y - mean) ** 2).mean(axis=-1, keepdims=True)
    yn = (y - mean) / np.sqrt(var + float(eps)) * _d(ln_w)[None] + _d(ln_b)[None]
    bonus = (_d(r) * _d(k) * _d(r_k)[None]).sum(axis=-1, keepdims=True)
    out = (yn + bonus * _d(v)) * _d(g)
    return out, y, s_out


GDN_NORM_EPS = 1e-12


def gdn_normalize(x):
    """x / max(||x||_2, 1e-12) over the last axis: the plain L2 normalisation,
    guarded so that a zero row (padding, a masked token) gives zeros."""
    x = _d(x)
    return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), GDN_NORM_EPS)


def gdn_decode_step(q, k, v, g, beta, s_in):
    """One token of a gated DeltaNet layer at matched head size N, computed as
    one WKV-7 step (the mapping of the rwkv-lab page, "Highlight result -- GDN
    in RWKV-7"). The gated delta rule S' = e^g S (I - beta k^ k^T) + beta v k^T
    expands to S diag(e^g) + (S (-k^)) (beta e^g k^)^T + v (beta k^)^T, i.e. a
    WKV-7 step with decay e^g on every key, a = -k^, b = beta e^g k^ and write
    key beta k^; its readout with r = q^, over sqrt(N), is GDN's output. q^ and
    k^ come from gdn_normalize.

    q, k [B, Hk, N] (key heads); v [B, H, N]; g, beta [B, H] (per value head);
    state [B, H, N, N]. Value head h reads key head h // (H / Hk): groups of
    consecutive value heads share a key head. Returns (out, s_out) in fp64."""
    q, k, v = _d(q), _d(k), _d(v)
    g, beta = _d(g), _d(beta)
    B, Hk, N = q.shape
    H = v.shape[1]
    kh = np.arange(H) // (H // Hk)
    qn = gdn_normalize(q)
    kn = gdn_normalize(k)
    r, kk = qn[:, kh], kn[:, kh]
    w = np.broadcast_to(np.exp(g)[..., None], (B, H, N))
    bt = beta[..., None]
    y, s_out = decode_step(r, w, bt * kk, v, -kk, kk * np.exp(g)[..., None] * bt, s_in)
    return np.asarray(y) / np.sqrt(N), s_out


def gdn_forward(q, k, v, g, beta, s0=None):
    """A sequence of gated DeltaNet tokens, each computed as the WKV-7 step
    of gdn_decode_step, token by token (rwkv-lab, "Highlight result -- GDN in
    RWKV-7"). q, k [B, T, Hk, N]; v [B, T, H, N]; g, beta [B, T, H]; s0
    [B, H, N, N] or None (zero). Returns (out [B, T, H, N], s_out) in fp64."""
    q, k, v = _d(q), _d(k), _d(v)
    g, beta = _d(g), _d(beta)
    B, T, Hk, N = q.shape
    H = v.shape[2]
    kh = np.arange(H) // (H // Hk)
    qn = gdn_normalize(q)[:, :, kh]
    kn = gdn_normalize(k)[:, :, kh]
    dec = np.exp(g)[..., None]
    bt = beta[..., None]
    w = np.broadcast_to(dec, (B, T, H, N))
    out = forward(qn, w, bt * kn, v, -kn, kn * dec * bt, s0=s0)
    return out["y"] / np.sqrt(N), out["s_out"]


def gdn_backward(q, k, v, g, beta, s0=None, dout=None, ds_out=None):
    """Reverse-mode gradients of L = sum <dout, out> + <ds_out, S_T> for
    gdn_forward (rwkv-lab, "Highlight result -- GDN in RWKV-7"), by the chain
    rule from the WKV-7 backward through the remap and the normalisation.
    gdn_forward runs the gated delta rule as a WKV-7 step whose decay is e^g
    on every key, whose a- and b-vectors are -k^ and beta e^g k^, whose
    written key is beta k^ (k_w) and whose read vector is q^, with the output
    scaled by 1/sqrt(N). Each of those is linear in k^ or q^, so:

        dq^ = dr;  dk^ = beta dk_w - da + beta e^g db
        dg = e^g (sum_j dw_j + beta sum_j db_j k^_j)
        dbeta = sum_j dk_w,j k^_j + e^g sum_j db_j k^_j
        x^ = x / max(|x|, 1e-12):  dx = (dx^ - x^ <x^, dx^>) / |x|  (|x| > 1e-12),
                                   dx = dx^ / 1e-12 otherwise

    Value heads that share a key head add their dq^, dk^. Shapes as in
    gdn_forward; dout [B, T, H, N] and ds_out [B, H, N, N] or None (zero).
    Returns dict dq, dk [B, T, Hk, N], dv [B, T, H, N], dg, dbeta [B, T, H]
    and ds0 [B, H, N, N], all fp64."""
    q, k, v = _d(q), _d(k), _d(v)
    g, beta = _d(g), _d(beta)
    B, T, Hk, N = q.shape
    H = v.shape[2]
    grp = H // Hk
    kh = np.arange(H) // grp
    qd = np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), GDN_NORM_EPS)
    kd = np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), GDN_NORM_EPS)
    qn, kn = q / qd, k / kd
    r, kk = qn[:, :, kh], kn[:, :, kh]
    dec = np.exp(g)[..., None]
    bt = beta[..., None]
    w = np.broadcast_to(dec, (B, T, H, N))
    dy = None if dout is None else _d(dout) / np.sqrt(N)
    gr = backward(r, w, bt * kk, v, -kk, kk * dec * bt, s0=s0, dy=dy, ds_out=ds_out)
    dkk = bt * gr["dk"] - gr["da"] + bt * dec * gr["db"]
    dg = np.exp(g) * (np.sum(gr["dw"], axis=-1) + beta * np.sum(gr["db"] * kk, axis=-1))
    dbeta = np.sum(gr["dk"] * kk, axis=-1) + np.exp(g) * np.sum(gr["db"] * kk, axis=-1)
    dqn = gr["dr"].reshape(B, T, Hk, grp, N).sum(axis=3)
    dkn = dkk.reshape(B, T, Hk, grp, N).sum(axis=3)

    def through_norm(xn, xd, dxn):
        proj = np.sum(xn * dxn, axis=-1, keepdims=True)
        return np.where(xd > GDN_NORM_EPS, (dxn - xn * proj) / xd, dxn / GDN_NORM_EPS)

    return {"dq": through_norm(qn, qd, dqn), "dk": through_norm(kn, kd, dkn), "dv": gr["dv"],
            "dg": dg, "dbeta": dbeta, "ds0": gr["ds0"]}
