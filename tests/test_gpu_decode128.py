"""GPU parity of the WKV-7 decode step at head size 128 (the matched head
size of the rwkv-lab page's GDN conversion target) against the fp64 oracle,
through the C ABI. Tolerances as at head size 64: 1e-5 for fp32 outputs and
every state, 2e-2 for bf16 y, 2e-3 for fp16."""
import numpy as np
import pytest

from linear_recurrent_lm_amd import synth
from oracle import oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N = 128
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
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def state(B, H, seed):
    return (0.1 * np.random.Generator(np.random.PCG64(seed)).standard_normal((B, H, N, N))).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("decay", ["mult", "log"])
def test_decode128_parity(W, dtype, decay):
    import torch
    inp = synth.make_inputs(5, 1, 3, N, seed=48, dtype=dtype, decay=decay)
    s0 = state(5, 3, 48)
    ts = [U.dev_stream(x[:, 0], dtype) for x in inp.streams()]
    y, s1 = W.wkv7_decode_step(*ts, U.dev_f32(s0), decay=decay)
    torch.cuda.synchronize()
    r, w, k, v, a, b = (x[:, 0].astype(np.float64) for x in inp.streams())
    if decay == "log":
        w = np.exp(w)
    ry, rs = O.decode_step(r, w, k, v, a, b, s0)
    assert unit_err(U.host(y), ry) <= TOL[dtype]
    assert U.unit_err_state(U.host(s1), rs) <= U.TOL_F32


def test_decode128_chain_equals_forward(W):
    """20 steps with the state in place equal the oracle's token-order forward
    over the same 20 tokens."""
    import torch
    B, T, H = 3, 20, 2
    inp = synth.make_inputs(B, T, H, N, seed=49, dtype="f32")
    s0 = state(B, H, 49)
    st = U.dev_f32(s0)
    ys = []
    for t in range(T):
        ts = [U.dev_f32(np.ascontiguousarray(x[:, t])) for x in inp.streams()]
        y, _ = W.wkv7_decode_step(*ts, st, s_out=st)
        ys.append(y)
    torch.cuda.synchronize()
    ref = O.forward(*inp.streams(), s0=s0)
    got = np.stack([U.host(y) for y in ys], axis=1)
    assert U.unit_err_dense(got, ref["y"]) <= U.TOL_F32
    assert U.unit_err_state(U.host(st), ref["s_out"]) <= U.TOL_F32


def test_decode128_workload_all_units(W):
    """B = 128, H = 32 at head size 128, bf16, in place: every unit."""
    import torch
    inp = synth.make_inputs(128, 1, 32, N, seed=50, dtype="bf16")
    s0 = state(128, 32, 50)
    ts = [U.dev_stream(x[:, 0], "bf16") for x in inp.streams()]
    st = U.dev_f32(s0)
    y, _ = W.wkv7_decode_step(*ts, st, s_out=st)
    torch.cuda.synchronize()
    ry, rs = O.decode_step(*(x[:, 0] for x in inp.streams()), s0)
    assert unit_err(U.host(y), ry) <= U.TOL_BF16_Y
    assert U.unit_err_state(U.host(st), rs) <= U.TOL_F32
