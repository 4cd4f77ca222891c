"""GPU parity of the gated DeltaNet decode step (wkv7_gdn_decode_step: one
token through the RWKV-7 remap, head size 128 or 64) against the fp64
oracle's gdn_decode_step, through the C ABI. Tolerances as for the WKV-7
decode step: 1e-5 for fp32 outputs and every state, 2e-2 for bf16 outputs,
2e-3 for fp16."""
import numpy as np
import pytest

from linear_recurrent_lm_amd import synth
from oracle import oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL = {"f32": U.TOL_F32, "bf16": U.TOL_BF16_Y, "f16": U.TOL_F16}


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def unit_err(x, ref):
    """[B, H, N]: unit = (b, h)."""
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def run(W, inp, dtype, in_place=False):
    import torch
    q, k, v = (U.dev_stream(x, dtype) for x in (inp.q, inp.k, inp.v))
    s_in = U.dev_f32(inp.s0)
    out, s_out = W.wkv7_gdn_decode_step(q, k, v, U.dev_f32(inp.g), U.dev_f32(inp.beta), s_in,
                                        s_out=s_in if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert s_out.data_ptr() == s_in.data_ptr()
    return U.host(out), U.host(s_out)


@pytest.mark.parametrize("N", [128, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gdn_decode_parity(W, N, dtype):
    inp = synth.make_gdn_inputs(3, 8, 4, N, seed=44, dtype=dtype)
    out, s_out = run(W, inp, dtype)
    ro, rs = O.gdn_decode_step(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert unit_err(out, ro) <= TOL[dtype]
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


def test_gdn_decode_in_place_one_head_per_key(W):
    inp = synth.make_gdn_inputs(5, 4, 4, 128, seed=45, dtype="f32")
    out, s_out = run(W, inp, "f32", in_place=True)
    ro, rs = O.gdn_decode_step(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert unit_err(out, ro) <= U.TOL_F32
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


def test_gdn_decode_workload_all_units(W):
    """GDN's layer geometry (32 value heads over 16 key heads, N = 128), bf16,
    B = 64: every unit."""
    inp = synth.make_gdn_inputs(64, 32, 16, 128, seed=46, dtype="bf16")
    out, s_out = run(W, inp, "bf16")
    ro, rs = O.gdn_decode_step(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert unit_err(out, ro) <= U.TOL_BF16_Y
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


def test_gdn_decode_chain(W):
    """Four steps with the state carried in place equal four oracle steps."""
    import torch
    B, H, Hk, N = 2, 4, 2, 128
    steps = [synth.make_gdn_inputs(B, H, Hk, N, seed=47 + t, dtype="f32") for t in range(4)]
    s_dev = U.dev_f32(steps[0].s0)
    s_ref = steps[0].s0.astype(np.float64)
    for inp in steps:
        q, k, v = (U.dev_f32(x) for x in (inp.q, inp.k, inp.v))
        out, _ = W.wkv7_gdn_decode_step(q, k, v, U.dev_f32(inp.g), U.dev_f32(inp.beta), s_dev,
                                        s_out=s_dev)
        ro, s_ref = O.gdn_decode_step(inp.q, inp.k, inp.v, inp.g, inp.beta, s_ref)
        torch.cuda.synchronize()
        assert unit_err(U.host(out), ro) <= U.TOL_F32
    assert U.unit_err_state(U.host(s_dev), s_ref) <= U.TOL_F32


def run_seq(W, inp, dtype):
    import torch
    q, k, v = (U.dev_stream(x, dtype) for x in (inp.q, inp.k, inp.v))
    s0 = None if inp.s0 is None else U.dev_f32(inp.s0)
    out, s_out = W.wkv7_gdn_forward(q, k, v, U.dev_f32(inp.g), U.dev_f32(inp.beta), s0)
    torch.cuda.synchronize()
    return U.host(out), U.host(s_out)


@pytest.mark.parametrize("N", [128, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gdn_forward_parity(W, N, dtype):
    """T = 37 tokens, two value heads per key head, with an initial state."""
    inp = synth.make_gdn_sequence(3, 37, 4, 2, N, seed=51, dtype=dtype, s0_std=0.1)
    out, s_out = run_seq(W, inp, dtype)
    ro, rs = O.gdn_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert U.unit_err_dense(out, ro) <= TOL[dtype]
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


@pytest.mark.parametrize("T", [1, 2, 16])
def test_gdn_forward_short_and_zero_state(W, T):
    inp = synth.make_gdn_sequence(2, T, 2, 2, 128, seed=52 + T, dtype="f32")
    out, s_out = run_seq(W, inp, "f32")
    ro, rs = O.gdn_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, None)
    assert U.unit_err_dense(out, ro) <= U.TOL_F32
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


def test_gdn_forward_equals_decode_steps(W):
    """The sequence call equals T decode steps with the state carried."""
    import torch
    inp = synth.make_gdn_sequence(2, 9, 4, 2, 128, seed=55, dtype="f32", s0_std=0.1)
    out, s_out = run_seq(W, inp, "f32")
    st = U.dev_f32(inp.s0)
    for t in range(9):
        o, _ = W.wkv7_gdn_decode_step(*(U.dev_f32(np.ascontiguousarray(x[:, t])) for x in (inp.q, inp.k, inp.v)),
                                      U.dev_f32(np.ascontiguousarray(inp.g[:, t])),
                                      U.dev_f32(np.ascontiguousarray(inp.beta[:, t])), st, s_out=st)
        torch.cuda.synchronize()
        assert unit_err(U.host(o), out[:, t]) <= U.TOL_F32
    assert U.unit_err_state(U.host(st), s_out) <= U.TOL_F32


def test_gdn_forward_prefill_sampled(W):
    """Prefill at GDN's layer geometry: B = 16, T = 1024, 32 value heads over
    16 key heads, N = 128, bf16; rows 0 and 15 (all heads) against the oracle."""
    inp = synth.make_gdn_sequence(16, 1024, 32, 16, 128, seed=56, dtype="bf16")
    out, s_out = run_seq(W, inp, "bf16")
    for b in (0, 15):
        sl = slice(b, b + 1)
        ro, rs = O.gdn_forward(inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl], inp.beta[sl], None)
        assert U.unit_err_dense(out[sl], ro) <= U.TOL_BF16_Y, b
        assert U.unit_err_state(s_out[sl], rs) <= U.TOL_F32, b


@pytest.mark.parametrize("N", [128, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_forward_strong_and_zero_decay(W, N, dtype):
    """Decays that drive the running decay product below 2^-60 within a few
    tokens (g = -30 at tokens 3..6), an exact zero decay (g = -inf at token
    11) and mild decays elsewhere. fp32 I/O runs token by token with the
    state divided by that product and folded back before it gets that small;
    bf16 I/O runs the chunk form, whose pair decays are products of e^g (zero
    included). out and the final state still match the oracle."""
    inp = synth.make_gdn_sequence(2, 40, 4, 2, N, seed=59, dtype=dtype, s0_std=0.1)
    inp.g[:, 3:7] = -30.0
    inp.g[:, 11] = -np.inf
    inp.g[:, 20:22] = -30.0
    out, s_out = run_seq(W, inp, dtype)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(s_out))
    ro, rs = O.gdn_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert U.unit_err_dense(out, ro) <= TOL[dtype]
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


@pytest.mark.parametrize("N", [128, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn_zero_q_and_k_rows(W, N, dtype):
    """All-zero k (token 5) and all-zero q (token 9) rows in the middle of a
    sequence, as padding or masked tokens give: the state stays finite, a zero
    k only decays it, a zero q outputs zero; the decode step agrees."""
    import torch
    inp = synth.make_gdn_sequence(2, 16, 4, 2, N, seed=57, dtype=dtype, s0_std=0.1)
    inp.k[:, 5] = 0.0
    inp.q[:, 9] = 0.0
    out, s_out = run_seq(W, inp, dtype)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(s_out))
    ro, rs = O.gdn_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.s0)
    assert U.unit_err_dense(out, ro) <= TOL[dtype]
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32
    assert np.max(np.abs(out[:, 9])) == 0.0
    dec = synth.make_gdn_inputs(2, 4, 2, N, seed=58, dtype="f32")
    dec.k[1] = 0.0
    dec.q[0] = 0.0
    o, s1 = run(W, dec, "f32")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s1))
    ro, rs = O.gdn_decode_step(dec.q, dec.k, dec.v, dec.g, dec.beta, dec.s0)
    assert unit_err(o, ro) <= U.TOL_F32
    assert U.unit_err_state(s1, rs) <= U.TOL_F32
    assert np.max(np.abs(o[0])) == 0.0
