"""wkv7_backward_noalloc (the backward on the library's static per-device
scratch, for callers that cannot allocate) against wkv7_backward with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller input than the first (so the scratch holds the first call's larger
contents), each bit-identical to the workspace entry point (same kernels,
same inputs); dense and segment mode; and the size limit."""
import numpy as np
import pytest

from linear_recurrent_lm_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

GRADS = ("dr", "dw", "dk", "dv", "da", "db", "ds0")


@pytest.fixture(scope="module")
def W():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_lm_amd import wkv7
    wkv7.lib()
    return wkv7


def _both(W, inp, segments=None):
    import torch
    ts = [U.dev_stream(getattr(inp, n), inp.dtype) for n in ("r", "w", "k", "v", "a", "b")]
    s0 = U.dev_f32(inp.s0)
    _, _, ckpt = W.wkv7_forward(*ts, s0, checkpoints=True, segments=segments)
    dy = U.dev_stream(inp.dy, inp.dtype)
    dso = U.dev_f32(inp.ds_out)
    ref = W.wkv7_backward(*ts, ckpt, dy, dso, segments=segments)
    got = W.wkv7_backward_noalloc(*ts, ckpt, dy, dso, segments=segments)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_backward_twice(W):
    import torch
    big = synth.make_inputs(2, 300, 8, 64, seed=71, dtype="bf16", s0_std=0.1, with_dy=True,
                            ds_out_std=0.1)
    small = synth.make_inputs(1, 70, 4, 64, seed=72, dtype="f32", s0_std=0.1, with_dy=True,
                              ds_out_std=0.1)
    for inp in (big, small):
        ref, got = _both(W, inp)
        for n in GRADS:
            assert torch.equal(ref[n], got[n]), n
            assert bool(torch.isfinite(got[n]).all()), n


def test_noalloc_segments(W):
    import torch
    lengths = np.array([5, 40, 17, 33], dtype=np.int32)
    flat, s0 = synth.make_segment_inputs(lengths, 3, 64, seed=73, dtype="bf16", s0_std=0.1, with_dy=True)
    T, st, ln = synth.packed_layout(lengths, 2)
    order, st_s, ln_s = synth.sorted_table(st, ln)
    inp = synth.scatter_segments(flat, lengths, st, 2, T, dtype="bf16")
    inp.s0 = s0[order]
    seg = W.Segments(2, T, st_s, ln_s, "cuda:0")
    ref, got = _both(W, inp, seg)
    for n in GRADS:
        assert torch.equal(ref[n], got[n]), n


def test_noalloc_refuses_beyond_the_scratch(W):
    """B=4, T=4096, H=32 needs 688 MiB of per-chunk results: refused before
    anything is launched."""
    inp_shape = (4, 4096, 32, 64)
    assert W.wkv7_workspace_bytes(4, 4096, 32, W.BF16) > W.STATIC_SCRATCH_BYTES
    import torch
    ts = [torch.zeros(inp_shape, device="cuda:0", dtype=torch.bfloat16) for _ in range(6)]
    ck = torch.zeros((4 * 256, 32, 64, 64), device="cuda:0", dtype=torch.float32)
    with pytest.raises(W.WKV7Error) as e:
        W.wkv7_backward_noalloc(*ts, ck)
    assert e.value.code == 3
