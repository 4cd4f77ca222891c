"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element. Small shapes span several 16-token
chunks and a ragged tail; the full-size workloads are checked on sampled
(sequence, head) units that the oracle computes one by one."""
import numpy as np
import pytest

from oracle import oracle as O
from linear_recurrent_lm_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def run_forward(W, inp, *, checkpoints=True, segments=None):
    import torch
    names = ("r", "w", "k", "v", "a", "b")
    ts = [U.dev_stream(getattr(inp, n), inp.dtype) for n in names]
    s0 = U.dev_f32(inp.s0)
    y, s_out, ckpt = W.wkv7_forward(*ts, s0, checkpoints=checkpoints, segments=segments)
    torch.cuda.synchronize()
    return ts, s0, y, s_out, ckpt


def ytol(dtype):
    return U.TOL_F32 if dtype == "f32" else U.TOL_BF16_Y


def gtol(dtype):
    return 1e-4 if dtype == "f32" else U.TOL_GRAD


# ------------------------------------------------------------------ forward

def test_forward_small_f32_workload(W):
    """B=1, T=64, H=1, fp32, zero state, seed 0: every output within 1e-5."""
    inp = synth.make_inputs(1, 64, 1, 64, seed=0, dtype="f32")
    _, _, y, s_out, ckpt = run_forward(W, inp)
    ref = O.forward(*inp.streams(), checkpoints=True)
    assert U.unit_err_dense(U.host(y), ref["y"]) <= U.TOL_F32
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_ckpt(U.host(ckpt), ref["ckpt"], [0], [4]) <= U.TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 33, 100])
def test_forward_shapes(W, T, dtype):
    B, H = 2, 3
    inp = synth.make_inputs(B, T, H, 64, seed=100 + T, dtype=dtype, s0_std=0.1)
    _, _, y, s_out, ckpt = run_forward(W, inp)
    ref = O.forward(*inp.streams(), s0=inp.s0, checkpoints=True)
    nc = -(-T // 16)
    assert U.unit_err_dense(U.host(y), ref["y"]) <= ytol(dtype)
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_ckpt(U.host(ckpt), ref["ckpt"], [0, nc], [nc, nc]) <= U.TOL_F32


def test_forward_closed_forms(W):
    """a = b = 0: w = 0 keeps only the last v k^T; w = 1 accumulates sum v k^T."""
    import torch
    B, T, H = 2, 37, 2
    inp = synth.make_inputs(B, T, H, 64, seed=7, dtype="f32", s0_std=1.0)
    r, k, v = inp.r.astype(np.float64), inp.k.astype(np.float64), inp.v.astype(np.float64)
    zeros = np.zeros_like(inp.r)
    for wval in (0.0, 1.0):
        inp2 = synth.Inputs("f32", inp.r, np.full_like(inp.w, wval), inp.k, inp.v, zeros, zeros,
                            s0=inp.s0)
        _, _, y, s_out, _ = run_forward(W, inp2, checkpoints=False)
        if wval == 0.0:
            y_ref = v * np.sum(k * r, axis=-1, keepdims=True)
            S_ref = np.einsum("bhi,bhj->bhij", v[:, -1], k[:, -1])
        else:
            St = inp.s0.astype(np.float64)[:, None] + np.cumsum(
                np.einsum("bthi,bthj->bthij", v, k), axis=1)
            y_ref = np.einsum("bthij,bthj->bthi", St, r)
            S_ref = St[:, -1]
        assert U.unit_err_dense(U.host(y), y_ref) <= U.TOL_F32
        assert U.unit_err_state(U.host(s_out), S_ref) <= U.TOL_F32


def _sampled_forward(W, B, T, H, seed, s0_std, n_units=6):
    inp = synth.make_inputs(B, T, H, 64, seed=seed, dtype="bf16", s0_std=s0_std)
    _, _, y, s_out, ckpt = run_forward(W, inp)
    yh, sh, ch = U.host(y), U.host(s_out), U.host(ckpt)
    nc = -(-T // 16)
    worst = {"y": 0.0, "s_out": 0.0, "ckpt": 0.0}
    for (b, h) in U.sample_units(B, H, n_units, seed):
        sl = [x[b:b + 1, :, h:h + 1] for x in inp.streams()]
        s0 = None if inp.s0 is None else inp.s0[b:b + 1, h:h + 1]
        ref = O.forward(*sl, s0=s0, checkpoints=True)
        worst["y"] = max(worst["y"], U.unit_err_dense(yh[b:b + 1, :, h:h + 1], ref["y"]))
        worst["s_out"] = max(worst["s_out"], U.unit_err_state(sh[b:b + 1, h:h + 1], ref["s_out"]))
        worst["ckpt"] = max(worst["ckpt"], U.unit_err_ckpt(
            ch[b * nc:(b + 1) * nc, h:h + 1], ref["ckpt"], [0], [nc]))
    return worst


def test_forward_d768_workload_sampled(W):
    """bf16, B=8, T=4096, H=12, zero state (the 12-layer D=768 shape)."""
    e = _sampled_forward(W, 8, 4096, 12, seed=1, s0_std=0.0)
    assert e["y"] <= U.TOL_BF16_Y and e["s_out"] <= U.TOL_F32 and e["ckpt"] <= U.TOL_F32, e


def test_forward_d2048_prefill_sampled(W):
    """bf16, B=16, T=1024, H=32, random initial state N(0, 0.1^2)."""
    e = _sampled_forward(W, 16, 1024, 32, seed=2, s0_std=0.1)
    assert e["y"] <= U.TOL_BF16_Y and e["s_out"] <= U.TOL_F32 and e["ckpt"] <= U.TOL_F32, e


def test_forward_training_workload_sampled(W):
    """bf16, B=4, T=4096, H=32 (128 units: two 32-row workgroups per unit,
    state waves split by key columns), random initial state: y, s_out and
    checkpoints on sampled units."""
    e = _sampled_forward(W, 4, 4096, 32, seed=3, s0_std=0.1)
    assert e["y"] <= U.TOL_BF16_Y and e["s_out"] <= U.TOL_F32 and e["ckpt"] <= U.TOL_F32, e


@pytest.mark.parametrize("H", [64, 128])
def test_workgroup_shapes_f32(W, H):
    """fp32, B=2, T=77: 128 units run the forward and the state-gradient sweep
    as two 32-row workgroups per unit with key-split state waves, 256 units as
    one 64-row workgroup; every unit, forward and backward, against the oracle."""
    B, T = 2, 77
    inp = synth.make_inputs(B, T, H, 64, seed=300 + H, dtype="f32", s0_std=0.1,
                            with_dy=True, ds_out_std=0.1)
    _, _, y, s_out, ckpt = run_forward(W, inp)
    ref = O.forward(*inp.streams(), s0=inp.s0, checkpoints=True)
    nc = -(-T // 16)
    assert U.unit_err_dense(U.host(y), ref["y"]) <= U.TOL_F32
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_ckpt(U.host(ckpt), ref["ckpt"], [0, nc], [nc, nc]) <= U.TOL_F32
    g, _ = run_backward(W, inp)
    gr = O.backward(*inp.streams(), s0=inp.s0, dy=inp.dy, ds_out=inp.ds_out)
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        assert U.unit_err_dense(g[n], gr[n]) <= 1e-4, n
    assert U.unit_err_state(g["ds0"], gr["ds0"]) <= 1e-4


@pytest.mark.parametrize("decay", ["mult", "log"])
@pytest.mark.parametrize("B,H", [(8, 32), (4, 32), (2, 3)])
def test_bf16_fast_and_slow_chunks(W, decay, B, H):
    """bf16 streams with a zero decay (1e-13 as a logarithm) in chunk 1 and
    decays of 2^-10 on some keys in chunk 3. With 256 units (B=8, H=32) the
    forward runs 64-row workgroups whose state products are three-piece bf16
    MFMAs; there a chunk whose decays are all at least 2^-6 builds its 16x16
    matrices from bf16 MFMA tiles of decay-scaled rows (chunks 0, 2 and the
    partial chunk 4), any other chunk from the split-point rows. With 128
    units (B=4, H=32) and 6 units (B=2, H=3) the forward runs 32- and 16-row
    workgroups on FP32 MFMA, every chunk from the split-point rows. Every
    unit's y, final state and checkpoints against the oracle, for both decay
    inputs."""
    import torch
    T = 77
    inp = synth.make_inputs(B, T, H, 64, seed=500, dtype="bf16", s0_std=0.1, decay=decay)
    if decay == "mult":
        inp.w[:, 21] = 0.0
        inp.w[:, 50, :, :5] = 2.0 ** -10
    else:
        inp.w[:, 21] = synth.round_bf16(np.float32(np.log(1e-13)))
        inp.w[:, 50, :, :5] = synth.round_bf16(np.float32(np.log(2.0 ** -10)))
    ts = [U.dev_stream(x, "bf16") for x in inp.streams()]
    y, s_out, ckpt = W.wkv7_forward(*ts, U.dev_f32(inp.s0), checkpoints=True, decay=decay)
    torch.cuda.synchronize()
    w = inp.w.astype(np.float64)
    dec = np.exp(w) if decay == "log" else w
    ref = O.forward(inp.r, dec, inp.k, inp.v, inp.a, inp.b, s0=inp.s0, checkpoints=True)
    nc = -(-T // 16)
    assert U.unit_err_dense(U.host(y), ref["y"]) <= U.TOL_BF16_Y
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    assert U.unit_err_ckpt(U.host(ckpt), ref["ckpt"], [b * nc for b in range(B)], [nc] * B) <= U.TOL_F32


def test_forward_deterministic(W):
    import torch
    inp = synth.make_inputs(2, 100, 4, 64, seed=9, dtype="bf16", s0_std=0.1)
    _, _, y1, s1, c1 = run_forward(W, inp)
    _, _, y2, s2, c2 = run_forward(W, inp)
    assert torch.equal(y1, y2) and torch.equal(s1, s2) and torch.equal(c1, c2)


# ------------------------------------------------------------------ backward

def run_backward(W, inp, segments=None):
    import torch
    ts, s0, y, s_out, ckpt = run_forward(W, inp, segments=segments)
    dy = U.dev_stream(inp.dy, inp.dtype) if inp.dy is not None else None
    dso = U.dev_f32(inp.ds_out)
    g = W.wkv7_backward(*ts, ckpt, dy, dso, segments=segments)
    torch.cuda.synchronize()
    return {k: (U.host(v) if v is not None else None) for k, v in g.items()}, ckpt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 16, 17, 40, 273])     # 273: 18 chunks, workgroups of 16 and 2
def test_backward_shapes(W, T, dtype):
    B, H = 2, 3
    inp = synth.make_inputs(B, T, H, 64, seed=200 + T, dtype=dtype, s0_std=0.1,
                            with_dy=True, ds_out_std=0.1)
    g, _ = run_backward(W, inp)
    ref = O.backward(*inp.streams(), s0=inp.s0, dy=inp.dy, ds_out=inp.ds_out)
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        assert U.unit_err_dense(g[n], ref[n]) <= gtol(dtype), n
    assert U.unit_err_state(g["ds0"], ref["ds0"]) <= gtol(dtype)


def test_backward_zero_and_tiny_decay(W):
    """w = 0 (a state reset) and w = 1e-12 inside chunks: gradients stay finite
    and match the oracle (the kernels clamp decay factors at 2^-30)."""
    B, T, H = 1, 50, 2
    inp = synth.make_inputs(B, T, H, 64, seed=31, dtype="f32", s0_std=0.2, with_dy=True,
                            ds_out_std=0.1)
    inp.w[0, 5] = 0.0
    inp.w[0, 21, 0, :9] = 0.0
    inp.w[0, 33:38] = 1e-12
    _, _, y, s_out, _ = run_forward(W, inp)
    ref = O.forward(*inp.streams(), s0=inp.s0)
    assert U.unit_err_dense(U.host(y), ref["y"]) <= U.TOL_F32
    assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
    g, _ = run_backward(W, inp)
    gr = O.backward(*inp.streams(), s0=inp.s0, dy=inp.dy, ds_out=inp.ds_out)
    for n in ("dr", "dw", "dk", "dv", "da", "db"):
        assert np.all(np.isfinite(g[n])), n
        assert U.unit_err_dense(g[n], gr[n]) <= 1e-4, n
    assert U.unit_err_state(g["ds0"], gr["ds0"]) <= 1e-4


def test_backward_no_upstream(W):
    """dy = NULL and ds_out = NULL give zero gradients everywhere."""
    inp = synth.make_inputs(1, 20, 2, 64, seed=5, dtype="f32", s0_std=0.1)
    g, _ = run_backward(W, inp)
    for n in ("dr", "dw", "dk", "dv", "da", "db", "ds0"):
        assert np.all(g[n] == 0), n


def test_backward_training_workload_sampled(W):
    """bf16, B=4, T=4096, H=32, zero state, dy ~ N(0,1): sampled units."""
    B, T, H = 4, 4096, 32
    inp = synth.make_inputs(B, T, H, 64, seed=3, dtype="bf16", with_dy=True)
    g, ckpt = run_backward(W, inp)
    ch = U.host(ckpt)
    nc = T // 16
    worst = {}
    for (b, h) in U.sample_units(B, H, 3, 3):
        sl = [x[b:b + 1, :, h:h + 1] for x in inp.streams()]
        dy = inp.dy[b:b + 1, :, h:h + 1]
        ref = O.backward(*sl, dy=dy)
        for n in ("dr", "dw", "dk", "dv", "da", "db"):
            worst[n] = max(worst.get(n, 0.0), U.unit_err_dense(g[n][b:b + 1, :, h:h + 1], ref[n]))
        worst["ds0"] = max(worst.get("ds0", 0.0), U.unit_err_state(g["ds0"][b:b + 1, h:h + 1],
                                                                    ref["ds0"]))
        fr = O.forward(*sl, checkpoints=True)
        worst["ckpt"] = max(worst.get("ckpt", 0.0), U.unit_err_ckpt(
            ch[b * nc:(b + 1) * nc, h:h + 1], fr["ckpt"], [0], [nc]))
    assert worst["ckpt"] <= U.TOL_F32, worst
    assert all(v <= U.TOL_GRAD for k, v in worst.items() if k != "ckpt"), worst


# ------------------------------------------------------------------ segments

def _segment_case(W, dtype, lengths, streams, H=3, s0_std=0.1):
    flat, s0 = synth.make_segment_inputs(lengths, H, 64, seed=11, dtype=dtype,
                                         s0_std=s0_std, with_dy=True)
    T_pad, st, ln = synth.packed_layout(lengths, streams)
    order, st_s, ln_s = synth.sorted_table(st, ln)
    packed = synth.scatter_segments(flat, lengths, st, streams, T_pad, dtype=dtype)
    packed.seq_start, packed.seq_len = st_s, ln_s
    packed.s0 = None if s0 is None else s0[order]
    return packed, T_pad, order


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segments_packed_and_padded(W, dtype):
    """Packed streams with resets and right-padded rows both match the oracle
    per sequence; NaN padding leaks nowhere; padding outputs are zero."""
    import torch
    lengths = np.array([5, 16, 33, 1, 20, 17, 8, 47], dtype=np.int32)
    H = 3
    results = []
    for layout in ("packed", "padded"):
        if layout == "packed":
            inp, T, order = _segment_case(W, dtype, lengths, 3, H)
            B = 3
        else:
            flat, s0 = synth.make_segment_inputs(lengths, H, 64, seed=11, dtype=dtype,
                                                 s0_std=0.1, with_dy=True)
            T = 64
            st, ln = synth.padded_layout(lengths, T)
            inp = synth.scatter_segments(flat, lengths, st, len(lengths), T, dtype=dtype)
            inp.s0 = s0
            order = np.arange(len(lengths))
            B = len(lengths)
        seg = W.Segments(B, T, inp.seq_start, inp.seq_len, "cuda:0")
        _, _, y, s_out, ckpt = run_forward(W, inp, segments=seg)
        ref = O.forward(*inp.streams(), s0=inp.s0, seq_start=inp.seq_start, seq_len=inp.seq_len,
                        checkpoints=True)
        yh = U.host(y)
        assert np.all(np.isfinite(yh))
        assert U.unit_err_segments(yh, ref["y"], inp.seq_start, inp.seq_len, T) <= ytol(dtype)
        covered = np.zeros(B * T, bool)
        for s_, l_ in zip(inp.seq_start, inp.seq_len):
            covered[s_:s_ + l_] = True
        assert np.all(yh.reshape(B * T, H, 64)[~covered] == 0)
        assert U.unit_err_state(U.host(s_out), ref["s_out"]) <= U.TOL_F32
        nch = (inp.seq_len + 15) // 16
        assert U.unit_err_ckpt(U.host(ckpt), ref["ckpt"], seg.host_ckpt, nch) <= U.TOL_F32
        dy = U.dev_stream(inp.dy, dtype)
        ts = [U.dev_stream(getattr(inp, n), dtype) for n in ("r", "w", "k", "v", "a", "b")]
        g = W.wkv7_backward(*ts, ckpt, dy, None, segments=seg)
        torch.cuda.synchronize()
        gr = O.backward(*inp.streams(), s0=inp.s0, dy=inp.dy, seq_start=inp.seq_start,
                        seq_len=inp.seq_len)
        for n in ("dr", "dw", "dk", "dv", "da", "db"):
            gh = U.host(g[n])
            assert np.all(np.isfinite(gh)), n
            assert np.all(gh.reshape(B * T, H, 64)[~covered] == 0), n
            assert U.unit_err_segments(gh, gr[n], inp.seq_start, inp.seq_len, T) <= gtol(dtype), n
        assert U.unit_err_state(U.host(g["ds0"]), gr["ds0"]) <= gtol(dtype)
        results.append((order, U.host(s_out)))
    # same sequences, same final states in both layouts
    (o1, s1), (o2, s2) = results
    inv = np.empty_like(o1); inv[o1] = np.arange(len(o1))
    np.testing.assert_allclose(s1[inv], s2, rtol=0, atol=1e-5 * np.abs(s2).max())


def test_segments_ragged_workload_sampled(W):
    """64 sequences, lengths ~ U[16, 2048], packed in 4 streams, H=32, bf16,
    zero initial states: sampled sequences against the oracle."""
    H = 32
    lengths = synth.ragged_lengths(64, 16, 2048, seed=4)
    inp, T, order = _segment_case(W, "bf16", lengths, 4, H, s0_std=0.0)
    seg = W.Segments(4, T, inp.seq_start, inp.seq_len, "cuda:0")
    _, _, y, s_out, _ = run_forward(W, inp, segments=seg, checkpoints=False)
    yh, sh = U.host(y), U.host(s_out)
    rng = np.random.default_rng(4)
    for q in list(rng.choice(len(lengths), 4, replace=False)) + [int(np.argmax(inp.seq_len))]:
        st, L = int(inp.seq_start[q]), int(inp.seq_len[q])
        b, t0 = divmod(st, T)
        h = int(rng.integers(H))
        sl = [x[b:b + 1, t0:t0 + L, h:h + 1] for x in inp.streams()]
        ref = O.forward(*sl)
        assert U.unit_err_dense(yh[b:b + 1, t0:t0 + L, h:h + 1], ref["y"]) <= U.TOL_BF16_Y
        assert U.unit_err_state(sh[q:q + 1, h:h + 1], ref["s_out"]) <= U.TOL_F32


# ------------------------------------------------------------------ decode

def test_decode_workload_all_units(W):
    """B=512, T=1, H=32, bf16 I/O, fp32 state N(0, 0.1^2): every unit."""
    import torch
    inp = synth.make_decode_inputs(512, 32, seed=4)
    ts = [U.dev_stream(x[:, 0], "bf16") for x in inp.streams()]
    s_in = U.dev_f32(inp.s0)
    y, s_out = W.wkv7_decode_step(*ts, s_in)
    torch.cuda.synchronize()
    yr, sr = O.decode_step(*[x[:, 0] for x in inp.streams()], inp.s0)
    yh = U.host(y)
    num = np.max(np.abs(yh - yr), axis=2); den = np.maximum(np.max(np.abs(yr), axis=2), 1e-30)
    assert float(np.max(num / den)) <= U.TOL_BF16_Y
    assert U.unit_err_state(U.host(s_out), sr) <= U.TOL_F32


def test_decode_in_place_and_chain_equals_forward(W):
    import torch
    B, T, H = 8, 21, 4
    inp = synth.make_inputs(B, T, H, 64, seed=12, dtype="f32", s0_std=0.1)
    ts = [U.dev_stream(x, "f32") for x in inp.streams()]
    y_f, s_f, _ = W.wkv7_forward(*ts, U.dev_f32(inp.s0))
    state = U.dev_f32(inp.s0).clone()
    ys = []
    for t in range(T):
        y, out = W.wkv7_decode_step(*[x[:, t].contiguous() for x in ts], state, s_out=state)
        assert out.data_ptr() == state.data_ptr()
        ys.append(y)
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=1)
    assert U.unit_err_dense(U.host(yd), U.host(y_f)) <= U.TOL_F32
    assert U.unit_err_state(U.host(state), U.host(s_f)) <= U.TOL_F32
