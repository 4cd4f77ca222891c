"""The Python binding checks every buffer it hands to the C ABI, the caller's
own outputs and workspaces included: the ABI receives bare pointers and
cannot see sizes, so a wrong shape, dtype, device or stride must be refused
before the call. Runs on the CPU: the compute entry points are replaced by a
recorder (no kernel can run), the size queries are the real library's."""
import pytest
import torch

from linear_recurrent_lm_amd import vocab_ce as VC
from linear_recurrent_lm_amd import wkv7 as W

COMPUTE = ("wkv7_forward", "wkv7_backward", "wkv7_decode_step", "wkv7_decode_step_fused",
           "wkv7_gdn_decode_step", "wkv7_gdn_forward", "vce_forward", "vce_backward")


class Recorder:
    """The real library for size queries; compute calls are recorded only."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name in COMPUTE:
            def rec(*args):
                self.calls.append((name, args))
                return 0
            return rec
        return getattr(self.real, name)


@pytest.fixture
def rec(monkeypatch):
    r = Recorder(W.lib())
    monkeypatch.setattr(W, "lib", lambda: r)
    monkeypatch.setattr(W, "_cuda", lambda t, name: None)
    monkeypatch.setattr(W, "_stream", lambda: None)
    return r


def streams(B=2, T=20, H=3, n=64, dtype=torch.bfloat16):
    return [torch.zeros(B, T, H, n, dtype=dtype) for _ in range(6)]


def test_forward_checks_caller_outputs(rec):
    ts = streams()
    W.wkv7_forward(*ts, checkpoints=True)                        # all allocated here: accepted
    assert len(rec.calls) == 1
    bad = [
        dict(y=torch.zeros(2, 20, 3, 64, dtype=torch.float32)),              # y dtype
        dict(y=torch.zeros(2, 20, 3, 32, dtype=torch.bfloat16)),             # y shape
        dict(s_out=torch.zeros(2, 3, 64, 32)),                               # s_out shape
        dict(s_out=torch.zeros(2, 3, 64, 64, dtype=torch.float64)),          # s_out dtype
        dict(s_out=torch.zeros(2, 3, 64, 128)[..., :64]),                    # s_out strided
        dict(ckpt=torch.zeros(3, 3, 64, 64), checkpoints=True),              # 2 slots per row needed
        dict(ckpt=torch.zeros(4, 3, 64, 64, dtype=torch.bfloat16), checkpoints=True),
        dict(s0=torch.zeros(2, 3, 64, 64, dtype=torch.bfloat16)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            W.wkv7_forward(*ts, **kw)
    assert len(rec.calls) == 1


def test_backward_checks_workspace_and_gradients(rec):
    ts = streams()
    ck = torch.zeros(4, 3, 64, 64)
    W.wkv7_backward(*ts, ck)
    assert len(rec.calls) == 1
    need = W.wkv7_workspace_bytes(2, 20, 3, W.BF16)
    grads = {n: torch.zeros(2, 20, 3, 64, dtype=torch.bfloat16) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    W.wkv7_backward(*ts, ck, grads=grads, workspace=torch.zeros(need, dtype=torch.uint8))
    assert len(rec.calls) == 2
    # the workspace byte count passed is numel * element size
    assert rec.calls[-1][1][-2] == need
    W.wkv7_backward(*ts, ck, workspace=torch.zeros(need // 4, dtype=torch.float32))
    assert rec.calls[-1][1][-2] == need
    with pytest.raises(ValueError):
        W.wkv7_backward(*ts, ck, workspace=torch.zeros(need * 2, dtype=torch.uint8)[::2])
    g = dict(grads, dk=torch.zeros(2, 20, 3, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        W.wkv7_backward(*ts, ck, grads=g)
    with pytest.raises(ValueError):
        W.wkv7_backward(*ts, ck, dy=torch.zeros(2, 20, 3, 64))
    with pytest.raises(ValueError):
        W.wkv7_backward(*ts, torch.zeros(3, 3, 64, 64))
    assert len(rec.calls) == 3


def test_decode_checks_y(rec):
    ts = [torch.zeros(4, 2, 64, dtype=torch.bfloat16) for _ in range(6)]
    s = torch.zeros(4, 2, 64, 64)
    W.wkv7_decode_step(*ts, s, s_out=s)
    assert len(rec.calls) == 1
    for y in (torch.zeros(4, 2, 64), torch.zeros(4, 2, 32, dtype=torch.bfloat16),
              torch.zeros(4, 2, 128, dtype=torch.bfloat16)[..., ::2]):
        with pytest.raises(ValueError):
            W.wkv7_decode_step(*ts, s, y=y)
    with pytest.raises(ValueError):
        W.wkv7_decode_step(*ts, s, s_out=torch.zeros(4, 2, 64, 32))
    assert len(rec.calls) == 1


def test_gdn_forward_checks_workspace(rec):
    q = torch.zeros(2, 5, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(2, 5, 4, 128, dtype=torch.bfloat16)
    g = torch.zeros(2, 5, 4)
    need = W.wkv7_gdn_workspace_bytes(2, 5, 2, 128)
    W.wkv7_gdn_forward(q, q.clone(), v, g, g.clone(), workspace=torch.zeros(need // 4))
    assert rec.calls[-1][1][-2] == need               # bytes, not elements
    with pytest.raises(ValueError):
        W.wkv7_gdn_forward(q, q.clone(), v, g, g.clone(), workspace=torch.zeros(need // 2)[::2])
    with pytest.raises(ValueError):
        W.wkv7_gdn_forward(q, q.clone(), v, g, g.clone(), out=torch.zeros(2, 5, 4, 128))
    assert len(rec.calls) == 1


def test_cross_entropy_checks_buffers(rec):
    h = torch.zeros(8, 64, dtype=torch.bfloat16)
    w = torch.zeros(16, 64, dtype=torch.bfloat16)
    t = torch.zeros(8, dtype=torch.int32)
    VC.vce_forward(h, w, t)
    assert len(rec.calls) == 1
    with pytest.raises(ValueError):
        VC.vce_forward(h, w, t, loss=torch.zeros(7))
    with pytest.raises(ValueError):
        VC.vce_forward(h, w, t, workspace=torch.zeros(64))      # workspaces are uint8
    with pytest.raises(ValueError):
        VC.vce_backward(h, w, t, torch.zeros(8), torch.zeros(8), dw=torch.zeros(16, 32))
    assert len(rec.calls) == 1


def test_host_tensors_are_refused():
    ts = streams()
    with pytest.raises(ValueError, match="device"):
        W.wkv7_forward(*ts)
