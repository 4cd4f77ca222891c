"""GPU parity of wkv7_forward at head size 128 (token-order kernel) against
the fp64 oracle, through the C ABI: dense batches with and without an initial
state and checkpoints, all three dtypes, log-decay input, packed and
right-padded segments, and the prefill shape on sampled rows. Tolerances as
at head size 64: 1e-5 for fp32 streams and every state and checkpoint, 2e-2
for bf16 y, 2e-3 for fp16."""
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


def run(W, inp, dtype, s0=True, ckpt=True, decay="mult"):
    import torch
    ts = [U.dev_stream(x, dtype) for x in inp.streams()]
    y, s_out, ck = W.wkv7_forward(*ts, U.dev_f32(inp.s0) if s0 else None, checkpoints=ckpt, decay=decay)
    torch.cuda.synchronize()
    return U.host(y), U.host(s_out), None if ck is None else U.host(ck)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 40])
def test_forward128_dense(W, dtype, T):
    inp = synth.make_inputs(2, T, 3, N, seed=60 + T, dtype=dtype, s0_std=0.1)
    y, s_out, ck = run(W, inp, dtype)
    ref = O.forward(*inp.streams(), s0=inp.s0, checkpoints=True)
    assert U.unit_err_dense(y, ref["y"]) <= TOL[dtype]
    assert U.unit_err_state(s_out, ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_state(ck, ref["ckpt"]) <= U.TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward128_log_decay_zero_state(W, dtype):
    inp = synth.make_inputs(3, 37, 2, N, seed=66, dtype=dtype, decay="log")
    y, s_out, _ = run(W, inp, dtype, s0=False, ckpt=False, decay="log")
    r, w, k, v, a, b = inp.streams()
    ref = O.forward(r, np.exp(w.astype(np.float64)), k, v, a, b)
    assert U.unit_err_dense(y, ref["y"]) <= TOL[dtype]
    assert U.unit_err_state(s_out, ref["s_out"]) <= U.TOL_F32


@pytest.mark.parametrize("layout", ["packed", "padded"])
def test_forward128_segments(W, layout):
    """Sequences with a state reset at each boundary, packed three to a row or
    right-padded one to a row (NaN padding): each equals the oracle, with its
    own initial state and checkpoints; outputs outside every sequence are 0."""
    import torch
    lengths = np.array([5, 16, 33, 1, 20, 17], dtype=np.int32)
    H = 2
    flat, s0 = synth.make_segment_inputs(lengths, H, N, seed=67, dtype="f32", s0_std=0.1)
    if layout == "packed":
        B, T = 2, 64                           # sequences 0-2 fill row 0, 3-5 row 1
        starts = []
        for i, L in enumerate(lengths):
            row, first = divmod(i, 3)
            starts.append(row * T + int(np.sum(lengths[row * 3:row * 3 + first])))
        st = np.array(starts, dtype=np.int32)
    else:
        B, T = len(lengths), 40
        st, _ = synth.padded_layout(lengths, T)
    inp = synth.scatter_segments(flat, lengths, st, B, T, dtype="f32")
    seg = W.Segments(B, T, inp.seq_start, inp.seq_len, "cuda:0")
    ts = [U.dev_stream(getattr(inp, n), "f32") for n in ("r", "w", "k", "v", "a", "b")]
    y, s_out, ck = W.wkv7_forward(*ts, U.dev_f32(s0), segments=seg, checkpoints=True)
    torch.cuda.synchronize()
    ref = O.forward(*inp.streams(), s0=s0, seq_start=inp.seq_start, seq_len=inp.seq_len,
                    checkpoints=True)
    yh = U.host(y)
    assert np.all(np.isfinite(yh))
    assert U.unit_err_segments(yh, ref["y"], inp.seq_start, inp.seq_len, T) <= U.TOL_F32
    covered = np.zeros(B * T, bool)
    for s_, l_ in zip(inp.seq_start, inp.seq_len):
        covered[s_:s_ + l_] = True
    assert np.all(yh.reshape(B * T, H, N)[~covered] == 0)
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    nch = (inp.seq_len + 15) // 16
    assert U.unit_err_ckpt(U.host(ck), ref["ckpt"], seg.host_ckpt, nch) <= U.TOL_F32


@pytest.mark.parametrize("decay", ["mult", "log"])
def test_forward128_zero_and_tiny_decay(W, decay):
    """Blocks whose decays are all at least 2^-6 run on a decay-normalised
    state; the others (a zero decay at token 5, 1e-12 at tokens 33..37, 2^-10
    on some keys at token 50) take the direct update. Both kinds, in both
    decay inputs, against the oracle: y, the final state and the checkpoints."""
    B, T, H = 2, 61, 2
    inp = synth.make_inputs(B, T, H, N, seed=69, dtype="f32", s0_std=0.2, decay=decay)
    vals = {5: 0.0, 33: 1e-12, 34: 1e-12, 35: 1e-12, 36: 1e-12, 37: 1e-12}
    for t, x in vals.items():
        inp.w[:, t] = np.log(x) if decay == "log" and x > 0 else (-1e30 if decay == "log" else x)
    inp.w[:, 50, :, :9] = np.log(2.0 ** -10) if decay == "log" else 2.0 ** -10
    y, s_out, ck = run(W, inp, "f32", decay=decay)
    w = inp.w.astype(np.float64)
    dec = np.exp(w) if decay == "log" else w
    ref = O.forward(inp.r, dec, inp.k, inp.v, inp.a, inp.b, s0=inp.s0, checkpoints=True)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(s_out))
    assert U.unit_err_dense(y, ref["y"]) <= U.TOL_F32
    assert U.unit_err_state(s_out, ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_state(ck, ref["ckpt"]) <= U.TOL_F32


def test_forward128_prefill_sampled(W):
    """Prefill shape B = 16, T = 1024, H = 32 at head size 128, bf16, random
    initial state: rows 0 and 15 (all heads) against the oracle."""
    inp = synth.make_inputs(16, 1024, 32, N, seed=68, dtype="bf16", s0_std=0.1)
    y, s_out, _ = run(W, inp, "bf16", ckpt=False)
    for b in (0, 15):
        sl = slice(b, b + 1)
        ref = O.forward(*(x[sl] for x in inp.streams()), s0=inp.s0[sl])
        assert U.unit_err_dense(y[sl], ref["y"]) <= U.TOL_BF16_Y, b
        assert U.unit_err_state(s_out[sl], ref["s_out"]) <= U.TOL_F32, b
