"""GPU parity of the I/O variants: fp16 activations (the model card's
"Transformers quickstart" names BF16/FP16/FP32 activations), w given as the
log of the decay (the wkv7 call on the rwkv-lab page, section "Highlight
result -- GDN in RWKV-7", takes GDN's log-decay), and fp32 gradients for
16-bit activations. Each is checked element by element against the fp64
oracle on the same seeded inputs; for a log-decay input the oracle runs on
decay = exp(w) and the expected gradient is decay * dL/d(decay)."""
import numpy as np
import pytest

from oracle import oracle as O
from linear_recurrent_lm_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

NAMES = ("dr", "dw", "dk", "dv", "da", "db")


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def _run(W, inp, *, grad_f32=False):
    import torch
    ts = [U.dev_stream(x, inp.dtype) for x in inp.streams()]
    s0 = U.dev_f32(inp.s0)
    y, s_out, ckpt = W.wkv7_forward(*ts, s0, checkpoints=True, decay=inp.decay)
    dy = U.dev_stream(inp.dy, inp.dtype)
    g = W.wkv7_backward(*ts, ckpt, dy, U.dev_f32(inp.ds_out), decay=inp.decay, grad_f32=grad_f32)
    torch.cuda.synchronize()
    return U.host(y), U.host(s_out), U.host(ckpt), {k: U.host(v) for k, v in g.items()}, g


def _oracle(inp):
    """Reference outputs and gradients for the stream values as the kernels read them."""
    w = inp.w.astype(np.float64)
    dec = np.exp(w) if inp.decay == "log" else w
    st = (inp.r, dec, inp.k, inp.v, inp.a, inp.b)
    f = O.forward(*st, s0=inp.s0, checkpoints=True)
    g = O.backward(*st, s0=inp.s0, dy=inp.dy, ds_out=inp.ds_out)
    if inp.decay == "log":
        g = dict(g)
        g["dw"] = dec * g["dw"]                  # d/d log(decay) = decay * d/d decay
    return f, g


def _check(inp, out, f, g, ytol, stol, gtol):
    y, s_out, ckpt, gh, _ = out
    B, T = inp.r.shape[:2]
    nc = -(-T // 16)
    assert U.unit_err_dense(y, f["y"]) <= ytol
    assert U.unit_err_state(s_out, f["s_out"]) <= stol
    assert U.unit_err_ckpt(ckpt, f["ckpt"], [b * nc for b in range(B)], [nc] * B) <= stol
    for n in NAMES:
        assert np.all(np.isfinite(gh[n])), n
        assert U.unit_err_dense(gh[n], g[n]) <= gtol, n
    assert U.unit_err_state(gh["ds0"], g["ds0"]) <= gtol


@pytest.mark.parametrize("T", [1, 17, 40, 100, 273])
def test_f16_forward_backward(W, T):
    inp = synth.make_inputs(2, T, 3, 64, seed=400 + T, dtype="f16", s0_std=0.1, with_dy=True,
                            ds_out_std=0.1)
    out = _run(W, inp)
    f, g = _oracle(inp)
    _check(inp, out, f, g, U.TOL_F16, U.TOL_F32, U.TOL_F16)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_log_decay_forward_backward(W, dtype):
    inp = synth.make_inputs(2, 45, 3, 64, seed=410, dtype=dtype, s0_std=0.1, with_dy=True,
                            ds_out_std=0.1, decay="log")
    # decays far below the kernels' 2^-30 clamp (w = e^-30, e^-60) and a full reset
    inp.w[0, 7, 1] = -30.0
    inp.w[1, 20:23] = -60.0
    out = _run(W, inp)
    f, g = _oracle(inp)
    ytol = {"f32": U.TOL_F32, "bf16": U.TOL_BF16_Y, "f16": U.TOL_F16}[dtype]
    gtol = {"f32": 1e-4, "bf16": U.TOL_GRAD, "f16": U.TOL_F16}[dtype]
    _check(inp, out, f, g, ytol, U.TOL_F32, gtol)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [50, 273])
def test_f32_gradients_for_16bit_inputs(W, dtype, T):
    """fp32 gradients of bf16/fp16 inputs: only the fp32 compute error remains,
    so they are held to the fp32 gradient bound."""
    import torch
    inp = synth.make_inputs(2, T, 3, 64, seed=420 + T, dtype=dtype, s0_std=0.1, with_dy=True,
                            ds_out_std=0.1)
    out = _run(W, inp, grad_f32=True)
    assert all(out[4][n].dtype == torch.float32 for n in NAMES)
    f, g = _oracle(inp)
    ytol = U.TOL_BF16_Y if dtype == "bf16" else U.TOL_F16
    _check(inp, out, f, g, ytol, U.TOL_F32, 1e-4)


@pytest.mark.parametrize("dtype,decay", [("f16", "mult"), ("f16", "log"), ("bf16", "log"), ("f32", "log")])
def test_decode_variants(W, dtype, decay):
    """One decode step at B=64, H=8 against the oracle's step on the same values."""
    import torch
    inp = synth.make_inputs(64, 1, 8, 64, seed=430, dtype=dtype, s0_std=0.1, decay=decay)
    ts = [U.dev_stream(x[:, 0], dtype) for x in inp.streams()]
    y, s_out = W.wkv7_decode_step(*ts, U.dev_f32(inp.s0), decay=decay)
    torch.cuda.synchronize()
    w = inp.w[:, 0].astype(np.float64)
    dec = np.exp(w) if decay == "log" else w
    yr, sr = O.decode_step(inp.r[:, 0], dec, inp.k[:, 0], inp.v[:, 0], inp.a[:, 0], inp.b[:, 0],
                           inp.s0)
    yh = U.host(y)
    num = np.max(np.abs(yh - yr), axis=2); den = np.maximum(np.max(np.abs(yr), axis=2), 1e-30)
    tol = {"f32": U.TOL_F32, "bf16": U.TOL_BF16_Y, "f16": U.TOL_F16}[dtype]
    assert float(np.max(num / den)) <= tol
    assert U.unit_err_state(U.host(s_out), sr) <= U.TOL_F32


def test_backward_gradient_dtypes_share_one_workspace(W):
    """bf16 streams hand the per-chunk results of the sweep to the gradient
    pass in bf16 for bf16 gradients and in fp32 for fp32 gradients. Calls of
    either kind, alternating on one workspace buffer, each match the oracle
    (bf16 gradients at the gradient bound, fp32 ones at 1e-4) and repeat
    bit for bit."""
    import torch
    inp = synth.make_inputs(2, 273, 3, 64, seed=440, dtype="bf16", s0_std=0.1, with_dy=True,
                            ds_out_std=0.1)
    ts = [U.dev_stream(x, "bf16") for x in inp.streams()]
    _, _, ckpt = W.wkv7_forward(*ts, U.dev_f32(inp.s0), checkpoints=True)
    dy, dso = U.dev_stream(inp.dy, "bf16"), U.dev_f32(inp.ds_out)
    ws = torch.empty(W.wkv7_workspace_bytes(2, 273, 3, W.BF16), dtype=torch.uint8, device="cuda:0")
    _, g_ref = _oracle(inp)
    first = {}
    for call, f32 in enumerate((False, True, False, True)):
        g = W.wkv7_backward(*ts, ckpt, dy, dso, grad_f32=f32, workspace=ws)
        torch.cuda.synchronize()
        h = {k: U.host(v) for k, v in g.items()}
        tol = 1e-4 if f32 else U.TOL_GRAD
        for n in NAMES:
            assert U.unit_err_dense(h[n], g_ref[n]) <= tol, (call, n)
        assert U.unit_err_state(h["ds0"], g_ref["ds0"]) <= 1e-4, call
        if f32 in first:
            for n in NAMES + ("ds0",):
                assert np.array_equal(h[n], first[f32][n]), (call, n)
        else:
            first[f32] = h
