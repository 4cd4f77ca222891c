"""Thin Python binding of the vocabulary cross-entropy in libwkv7.so (the C
ABI in include/vocab_ce.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the launch stream, outputs and the workspace are allocated
with torch.empty when the caller does not pass them. The loss, its lse and
both gradients are computed by the library's HIP kernels; if the library is
missing this module raises instead of computing anything.

Layouts: h [M, D] bf16, w [V, D] bf16, targets [M] int32 (values outside
[0, V) mark pad rows), loss / lse / dloss [M] fp32, dh [M, D] fp32,
dw [V, D] fp32, all contiguous on one device.
"""
from __future__ import annotations

import ctypes

from . import wkv7 as _W


def _check(fn, code):
    if code != 0:
        raise _W.WKV7Error(fn, code)


def vce_forward_workspace_bytes(M: int, D: int, V: int) -> int:
    out = ctypes.c_size_t(0)
    _check("vce_forward_workspace_bytes",
           _W.lib().vce_forward_workspace_bytes(M, D, V, ctypes.byref(out)))
    return out.value


def vce_backward_workspace_bytes(M: int, D: int, V: int, vocab_chunk: int) -> int:
    out = ctypes.c_size_t(0)
    _check("vce_backward_workspace_bytes",
           _W.lib().vce_backward_workspace_bytes(M, D, V, vocab_chunk, ctypes.byref(out)))
    return out.value


def _inputs(h, w, targets):
    torch = _W._torch()
    dev = h.device
    _W._cuda(h, "h")
    M, D = h.shape
    V = w.shape[0]
    _W._req(h, "h", dev, torch.bfloat16, (M, D))
    _W._req(w, "w", dev, torch.bfloat16, (V, D))
    _W._req(targets, "targets", dev, torch.int32, (M,))
    return torch, dev, M, D, V


def _workspace(torch, dev, need, workspace):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _W._req(workspace, "workspace", dev, torch.uint8)
    return workspace


def vce_forward(h, w, targets, *, loss=None, lse=None, workspace=None):
    """Returns (loss [M], lse [M]) in fp32."""
    torch, dev, M, D, V = _inputs(h, w, targets)
    loss = torch.empty(M, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(M, dtype=torch.float32, device=dev) if lse is None else lse
    _W._req(loss, "loss", dev, torch.float32, (M,))
    _W._req(lse, "lse", dev, torch.float32, (M,))
    ws = _workspace(torch, dev, vce_forward_workspace_bytes(M, D, V), workspace)
    _check("vce_forward", _W.lib().vce_forward(
        M, D, V, _W._ptr(h), _W._ptr(w), _W._ptr(targets), _W._ptr(loss), _W._ptr(lse),
        _W._ptr(ws), _W._nbytes(ws), _W._stream()))
    return loss, lse


def vce_backward(h, w, targets, lse, dloss, *, vocab_chunk: int = 16384, dh=None, dw=None,
                 workspace=None):
    """Returns (dh [M, D], dw [V, D]) in fp32; the vocabulary is processed vocab_chunk rows at a time."""
    torch, dev, M, D, V = _inputs(h, w, targets)
    _W._req(lse, "lse", dev, torch.float32, (M,))
    _W._req(dloss, "dloss", dev, torch.float32, (M,))
    dh = torch.empty(M, D, dtype=torch.float32, device=dev) if dh is None else dh
    dw = torch.empty(V, D, dtype=torch.float32, device=dev) if dw is None else dw
    _W._req(dh, "dh", dev, torch.float32, (M, D))
    _W._req(dw, "dw", dev, torch.float32, (V, D))
    ws = _workspace(torch, dev, vce_backward_workspace_bytes(M, D, V, vocab_chunk), workspace)
    _check("vce_backward", _W.lib().vce_backward(
        M, D, V, vocab_chunk, _W._ptr(h), _W._ptr(w), _W._ptr(targets), _W._ptr(lse),
        _W._ptr(dloss), _W._ptr(dh), _W._ptr(dw), _W._ptr(ws), _W._nbytes(ws), _W._stream()))
    return dh, dw
