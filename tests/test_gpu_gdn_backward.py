"""GPU parity of wkv7_gdn_backward (gated DeltaNet through the RWKV-7 remap)
against the fp64 oracle's gdn_backward, through the C ABI: both head sizes,
all three dtypes, an initial state with gradients on the output and on the
final state, no upstream gradient, zero q and k rows (the normalisation's
1e-12 floor), and GDN's layer geometry on sampled rows. The remapped streams
and every intermediate are fp32, so fp32 results (dg, dbeta, ds0 always;
dq, dk, dv for fp32 inputs) are held to 1e-4 per unit; 16-bit dq, dk, dv to
the gradient tolerances (5e-2 bf16, 2e-3 fp16)."""
import numpy as np
import pytest

from linear_recurrent_lm_amd import synth
from oracle import oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": U.TOL_GRAD, "f16": U.TOL_F16}
TOL_F32_GRAD = 1e-4


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def unit_err_scalar(x, ref):
    """[B, T, H]: unit = (b, h) over the tokens."""
    num = np.max(np.abs(x - ref), axis=1)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(num / den))


def upstream(inp, dtype, seed, dout=True, ds_out=True):
    rng = np.random.default_rng(seed)
    B, T, H, N = inp.v.shape
    do = synth.round_to(rng.standard_normal((B, T, H, N), dtype=np.float32), dtype) if dout else None
    dso = (rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(0.1)) if ds_out else None
    return do, dso


def run(W, inp, dtype, dout, ds_out):
    import torch
    q, k, v = (U.dev_stream(x, dtype) for x in (inp.q, inp.k, inp.v))
    s0 = None if inp.s0 is None else U.dev_f32(inp.s0)
    g = W.wkv7_gdn_backward(q, k, v, U.dev_f32(inp.g), U.dev_f32(inp.beta), s0,
                            None if dout is None else U.dev_stream(dout, dtype),
                            None if ds_out is None else U.dev_f32(ds_out))
    torch.cuda.synchronize()
    return {n: U.host(t) for n, t in g.items()}


def check(g, ref, dtype):
    for n in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(g[n])), n
        assert U.unit_err_dense(g[n], ref[n]) <= TOL[dtype], n
    for n in ("dg", "dbeta"):
        assert unit_err_scalar(g[n], ref[n]) <= TOL_F32_GRAD, n
    assert U.unit_err_state(g["ds0"], ref["ds0"]) <= TOL_F32_GRAD


@pytest.mark.parametrize("N", [128, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gdn_backward_parity(W, N, dtype):
    """T = 37 tokens (two full chunks and a ragged one), two value heads per
    key head, initial state, gradients on out and on the final state."""
    inp = synth.make_gdn_sequence(2, 37, 4, 2, N, seed=61, dtype=dtype, s0_std=0.1)
    dout, ds_out = upstream(inp, dtype, 62)
    g = run(W, inp, dtype, dout, ds_out)
    ref = O.gdn_backward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0, dout, ds_out)
    check(g, ref, dtype)


@pytest.mark.parametrize("T", [1, 16, 17])
def test_gdn_backward_lengths_zero_state(W, T):
    """One key head per value head, zero initial state, gradient on out only."""
    inp = synth.make_gdn_sequence(2, T, 3, 3, 128, seed=63 + T, dtype="f32")
    dout, _ = upstream(inp, "f32", 64, ds_out=False)
    g = run(W, inp, "f32", dout, None)
    ref = O.gdn_backward(inp.q, inp.k, inp.v, inp.g, inp.beta, None, dout, None)
    check(g, ref, "f32")


def test_gdn_backward_no_upstream(W):
    """dout = NULL and ds_out = NULL give zero gradients everywhere."""
    inp = synth.make_gdn_sequence(1, 20, 2, 1, 128, seed=65, dtype="f32", s0_std=0.1)
    g = run(W, inp, "f32", None, None)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "ds0"):
        assert np.all(g[n] == 0), n


@pytest.mark.parametrize("N", [128, 64])
def test_gdn_backward_zero_q_and_k_rows(W, N):
    """All-zero k (token 5) and q (token 9) rows: the normalisation's floor
    makes their gradients dx^ / 1e-12, which the oracle gives too."""
    inp = synth.make_gdn_sequence(2, 16, 4, 2, N, seed=66, dtype="f32", s0_std=0.1)
    inp.k[:, 5] = 0.0
    inp.q[:, 9] = 0.0
    dout, ds_out = upstream(inp, "f32", 67)
    g = run(W, inp, "f32", dout, ds_out)
    ref = O.gdn_backward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0, dout, ds_out)
    check(g, ref, "f32")
    assert np.max(np.abs(g["dk"][:, 5])) > 1e6      # the floor's 1/1e-12 scale


def test_gdn_backward_prefill_sampled(W):
    """GDN's layer geometry: B = 16, T = 1024, 32 value heads over 16 key
    heads, N = 128, bf16; rows 0 and 15 (all heads) against the oracle."""
    inp = synth.make_gdn_sequence(16, 1024, 32, 16, 128, seed=68, dtype="bf16")
    dout, _ = upstream(inp, "bf16", 69, ds_out=False)
    g = run(W, inp, "bf16", dout, None)
    for b in (0, 15):
        sl = slice(b, b + 1)
        ref = O.gdn_backward(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl], inp.beta[sl], None, dout[sl], None)
        sub = {n: g[n][sl] for n in g}
        check(sub, ref, "bf16")
