"""C-ABI checks of the vocabulary cross-entropy entry points that need no GPU:
the workspace queries and the argument validation, which must reject bad
sizes, pointers, alignments, overlaps and short workspaces with the
documented status codes before touching the HIP runtime."""
import ctypes

import pytest

from linear_recurrent_lm_amd import vocab_ce as C
from linear_recurrent_lm_amd import wkv7 as W

INVALID, UNSUPPORTED, WS = 1, 2, 3

# Fake, widely spaced, 16-byte aligned device addresses: validation must fail
# on the argument under test before any of these could be dereferenced.
P = [ctypes.c_void_p((q + 1) << 40) for q in range(12)]
BIG = 1 << 38


def fwd(M=300, D=128, V=1000, h=P[0], w=P[1], t=P[2], loss=P[3], lse=P[4], ws=P[5], nbytes=BIG):
    return W.lib().vce_forward(M, D, V, h, w, t, loss, lse, ws, nbytes, None)


def bwd(M=300, D=128, V=1000, chunk=256, h=P[0], w=P[1], t=P[2], lse=P[3], dl=P[4], dh=P[5],
        dw=P[6], ws=P[7], nbytes=BIG):
    return W.lib().vce_backward(M, D, V, chunk, h, w, t, lse, dl, dh, dw, ws, nbytes, None)


def test_declared_and_exported():
    names = set(W.declared_functions())
    want = {"vce_forward", "vce_backward", "vce_forward_workspace_bytes",
            "vce_backward_workspace_bytes"}
    assert want <= names
    for n in want:
        assert hasattr(W.lib(), n)


def test_workspace_queries():
    # forward: one (max, sum) pair per row and split plus the target logits
    assert C.vce_forward_workspace_bytes(16384, 2048, 65536) >= 16384 * 8 + 16384 * 4
    # backward: W^T, h^T, and G and G^T of one vocabulary chunk; vocabulary and
    # token rows padded to multiples of 256
    Vp, Mp, Vcp, D = 65536, 16384, 16384, 2048
    want = 2 * (D * Vp + D * Mp + 2 * Mp * Vcp)
    assert C.vce_backward_workspace_bytes(16384, D, 65536, 16384) == want
    # the chunk is rounded up to whole 256-row tiles and capped at V
    assert (C.vce_backward_workspace_bytes(100, 64, 1000, 4096)
            == 2 * (64 * 1024 + 64 * 256 + 2 * 256 * 1024))
    assert (C.vce_backward_workspace_bytes(100, 64, 1000, 300)
            == 2 * (64 * 1024 + 64 * 256 + 2 * 256 * 512))
    # a smaller chunk needs less
    assert (C.vce_backward_workspace_bytes(16384, D, 65536, 4096)
            < C.vce_backward_workspace_bytes(16384, D, 65536, 16384))


@pytest.mark.parametrize("M,D,V", [(0, 128, 10), (-1, 128, 10), ((1 << 28) + 1, 128, 10),
                                   (4, 0, 10), (4, 96, 10), (4, 32, 10), (4, 65600, 10),
                                   (4, 128, 0), (4, 128, (1 << 24) + 1)])
def test_bad_sizes(M, D, V):
    assert fwd(M=M, D=D, V=V) == INVALID
    assert bwd(M=M, D=D, V=V) == INVALID
    with pytest.raises(W.WKV7Error):
        C.vce_forward_workspace_bytes(M, D, V)
    with pytest.raises(W.WKV7Error):
        C.vce_backward_workspace_bytes(M, D, V, 64)


def test_forward_rejects_bad_pointers():
    for name in ("h", "w", "t", "loss", "lse", "ws"):
        assert fwd(**{name: None}) == INVALID, name
    assert fwd(h=ctypes.c_void_p(P[0].value + 8)) == INVALID      # bf16 operands: 16-byte aligned
    assert fwd(w=ctypes.c_void_p(P[1].value + 4)) == INVALID
    assert fwd(loss=ctypes.c_void_p(P[3].value + 2)) == INVALID
    assert fwd(ws=ctypes.c_void_p(P[5].value + 4)) == INVALID
    assert fwd(lse=ctypes.c_void_p(P[3].value + 64)) == INVALID    # overlaps loss
    assert fwd(loss=ctypes.c_void_p(P[0].value + 256)) == INVALID  # overlaps h
    assert fwd(ws=ctypes.c_void_p(P[1].value + 4096)) == INVALID   # overlaps w
    need = C.vce_forward_workspace_bytes(300, 128, 1000)
    assert fwd(nbytes=need - 1) == WS


def test_backward_rejects_bad_arguments():
    assert bwd(chunk=0) == INVALID
    for name in ("h", "w", "t", "lse", "dl", "dh", "dw", "ws"):
        assert bwd(**{name: None}) == INVALID, name
    assert bwd(dh=ctypes.c_void_p(P[5].value + 2)) == INVALID
    assert bwd(h=ctypes.c_void_p(P[0].value + 8)) == INVALID
    assert bwd(dw=ctypes.c_void_p(P[5].value + 1024)) == INVALID   # overlaps dh
    assert bwd(dh=ctypes.c_void_p(P[0].value + 1024)) == INVALID   # overlaps h
    assert bwd(ws=ctypes.c_void_p(P[6].value + 4096)) == INVALID   # overlaps dw
    need = C.vce_backward_workspace_bytes(300, 128, 1000, 256)
    assert bwd(nbytes=need - 1) == WS
    # grids beyond 2^22 workgroups are refused: gradient tiles (rows x chunk),
    # dh (rows x width) and dW (chunk x width)
    assert bwd(M=1 << 26, V=1 << 24, chunk=1 << 24) == INVALID
    assert bwd(M=1 << 28, D=65536, V=256, chunk=256) == INVALID
    assert bwd(M=256, D=65536, V=1 << 24, chunk=1 << 24) == INVALID
    with pytest.raises(W.WKV7Error):
        C.vce_backward_workspace_bytes(1 << 28, 65536, 256, 256)
    # the largest grid that is still allowed: 2^14 row tiles x 2^8 vocabulary tiles
    assert C.vce_backward_workspace_bytes(1 << 22, 64, 1 << 16, 1 << 16) > 0
