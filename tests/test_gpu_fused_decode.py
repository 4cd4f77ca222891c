"""GPU parity of the fused decode step (state update carried through the
per-head GroupNorm, the bonus and the output gate) against the fp64 oracle's
reading of the epilogue, through the C ABI. The gate, affine and bonus
weights are seeded inputs; the gate is rounded to the stream dtype first."""
import numpy as np
import pytest

from oracle import oracle as O
from linear_recurrent_lm_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL = {"f32": U.TOL_F32, "bf16": U.TOL_BF16_Y, "f16": U.TOL_F16}
EPS = 64e-5


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def epilogue_inputs(B, H, dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed + 3000))
    g = synth.round_to(rng.uniform(0.0, 2.0, size=(B, H, 64)).astype(np.float32), dtype)
    ln_w = (1.0 + 0.3 * rng.standard_normal((H, 64))).astype(np.float32)
    ln_b = (0.2 * rng.standard_normal((H, 64))).astype(np.float32)
    r_k = (0.5 * rng.standard_normal((H, 64))).astype(np.float32)
    return g, ln_w, ln_b, r_k


def unit_err(x, ref):
    """[B, H, N]: unit = (b, h)."""
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def run(W, inp, dtype, params, *, want_y=True, decay="mult", in_place=False):
    import torch
    ts = [U.dev_stream(x[:, 0], dtype) for x in inp.streams()]
    g, ln_w, ln_b, r_k = params
    s_in = U.dev_f32(inp.s0)
    out, s_out, y = W.wkv7_decode_step_fused(
        *ts, s_in, U.dev_stream(g, dtype), U.dev_f32(ln_w), U.dev_f32(ln_b), U.dev_f32(r_k), EPS,
        s_out=s_in if in_place else None, want_y=want_y, decay=decay)
    torch.cuda.synchronize()
    if in_place:
        assert s_out.data_ptr() == s_in.data_ptr()
    return U.host(out), U.host(s_out), None if y is None else U.host(y)


def oracle(inp, params, decay="mult"):
    r, w, k, v, a, b = (x[:, 0].astype(np.float64) for x in inp.streams())
    if decay == "log":
        w = np.exp(w)
    return O.decode_step_fused(r, w, k, v, a, b, inp.s0, *params, EPS)


def test_fused_decode_workload_all_units(W):
    """B=512, H=32, bf16 I/O, fp32 state N(0, 0.1^2): every unit."""
    inp = synth.make_decode_inputs(512, 32, seed=4)
    params = epilogue_inputs(512, 32, "bf16", 4)
    out, s_out, y = run(W, inp, "bf16", params)
    ro, ry, rs = oracle(inp, params)
    assert unit_err(out, ro) <= U.TOL_BF16_Y
    assert unit_err(y, ry) <= U.TOL_BF16_Y
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("want_y", [True, False])
def test_fused_decode_dtypes(W, dtype, want_y):
    inp = synth.make_decode_inputs(9, 5, seed=41, dtype=dtype)
    params = epilogue_inputs(9, 5, dtype, 41)
    out, s_out, y = run(W, inp, dtype, params, want_y=want_y)
    ro, ry, rs = oracle(inp, params)
    assert unit_err(out, ro) <= TOL[dtype]
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32
    assert (y is None) != want_y
    if want_y:
        assert unit_err(y, ry) <= TOL[dtype]


def test_fused_decode_log_decay_in_place(W):
    inp = synth.make_inputs(6, 1, 4, 64, seed=42, dtype="f32", decay="log")
    inp.s0 = (0.1 * np.random.Generator(np.random.PCG64(42)).standard_normal((6, 4, 64, 64))).astype(np.float32)
    params = epilogue_inputs(6, 4, "f32", 42)
    out, s_out, y = run(W, inp, "f32", params, decay="log", in_place=True)
    ro, ry, rs = oracle(inp, params, decay="log")
    assert unit_err(out, ro) <= U.TOL_F32
    assert unit_err(y, ry) <= U.TOL_F32
    assert U.unit_err_state(s_out, rs) <= U.TOL_F32


def test_fused_decode_graph_replay(W):
    """K fused steps (state updated in place) captured in one graph: every
    replay, with eager work and synchronisations between replays, equals the
    eager run of the same steps."""
    import torch
    B, H, K = 16, 8, 4
    inp = synth.make_inputs(B, K, H, 64, seed=43, dtype="bf16")
    s0 = (0.1 * np.random.Generator(np.random.PCG64(43)).standard_normal((B, H, 64, 64))).astype(np.float32)
    g, ln_w, ln_b, r_k = (U.dev_stream(epilogue_inputs(B, H, "bf16", 43)[0], "bf16"),
                          *[U.dev_f32(x) for x in epilogue_inputs(B, H, "bf16", 43)[1:]])
    steps = [[U.dev_stream(x[:, t], "bf16") for x in inp.streams()] for t in range(K)]
    state0 = U.dev_f32(s0)

    def run_steps(state, outs):
        for t in range(K):
            W.wkv7_decode_step_fused(*steps[t], state, g, ln_w, ln_b, r_k, EPS, s_out=state, out=outs[t])

    eager_state = state0.clone()
    eager_outs = [torch.empty_like(steps[0][0]) for _ in range(K)]
    run_steps(eager_state, eager_outs)
    torch.cuda.synchronize()
    want = [U.host(o) for o in eager_outs] + [U.host(eager_state)]

    state = state0.clone()
    outs = [torch.empty_like(steps[0][0]) for _ in range(K)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm the capture stream once
        run_steps(state, outs)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(state, outs)
    for rep in range(3):
        state.copy_(state0)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [U.host(o) for o in outs] + [U.host(state)]
        for t in range(K):
            assert np.array_equal(got[t], want[t]), (rep, t)
        assert np.array_equal(got[K], want[K]), rep
        # eager work between replays
        run_steps(eager_state.copy_(state0), eager_outs)
        torch.cuda.synchronize()
