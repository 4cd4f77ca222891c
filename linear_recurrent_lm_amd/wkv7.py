"""Thin Python binding of libwkv7.so (the C ABI in include/wkv7.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the launch stream, outputs are allocated with torch.empty.
Every step of the recurrence runs in the library's HIP kernels; if the
library is missing this module raises instead of computing anything.

Functions carry the C names (wkv7_forward, wkv7_backward, wkv7_decode_step,
...). Layouts: streams [B, T, H, 64] (fp32, bf16 or fp16, contiguous), states
[S, H, 64, 64] fp32, checkpoints [slots, H, 64, 64] fp32. decay="log" passes
w as log(decay); grad_f32=True writes the gradients in fp32.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# WKV7_LIBRARY names another build of the same library (the host-only
# AddressSanitizer build the CPU tests use); by default the in-tree one.
LIB_PATH = os.environ.get("WKV7_LIBRARY") or os.path.join(HERE, "libwkv7.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "wkv7.h")

N = 64
CHUNK = 16
F32, BF16, F16 = 0, 1, 2
DECAY = {"mult": 0, "log": 1}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "HIP runtime error"}


class WKV7Error(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({code})")
        self.code = code


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("dtype", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("seq_start", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("seq_ckpt", ctypes.c_void_p), ("ckpt_slots", ctypes.c_int32),
                ("decay", ctypes.c_int32), ("grad_f32", ctypes.c_int32)]


_lib = None


def declared_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        names |= set(re.findall(r"\b((?:wkv7|vce)_[a-z_]+)\s*\(", open(path).read()))
    return sorted(names)


def lib():
    """Load libwkv7.so (built by linear_recurrent_lm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run python -m linear_recurrent_lm_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dptr = ctypes.POINTER(Desc)
        L.wkv7_forward.argtypes = [dptr] + [vp] * 11
        L.wkv7_backward.argtypes = [dptr] + [vp] * 16 + [vp, sz, vp]
        L.wkv7_backward_noalloc.argtypes = [dptr] + [vp] * 17
        L.wkv7_decode_step.argtypes = [i32, i32, i32, i32, i32] + [vp] * 10
        L.wkv7_decode_step_fused.argtypes = ([i32, i32, i32, i32, i32] + [vp] * 12
                                             + [ctypes.c_float, vp, vp, vp])
        L.wkv7_checkpoint_slots.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_int64)]
        L.wkv7_workspace_bytes.argtypes = [dptr, ctypes.POINTER(ctypes.c_size_t)]
        L.wkv7_segments_check.argtypes = [i32, i32, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_int64)]
        L.wkv7_status_string.argtypes = [i32]
        L.wkv7_status_string.restype = ctypes.c_char_p
        L.wkv7_abi_version.restype = i32
        L.wkv7_gdn_decode_step.argtypes = [i32] * 5 + [vp] * 9
        L.wkv7_gdn_workspace_bytes.argtypes = [i32] * 4 + [ctypes.POINTER(sz)]
        L.wkv7_gdn_forward.argtypes = [i32] * 6 + [vp] * 9 + [sz, vp]
        L.wkv7_gdn_backward_workspace_bytes.argtypes = [i32] * 5 + [ctypes.POINTER(sz)]
        L.wkv7_gdn_backward.argtypes = [i32] * 6 + [vp] * 15 + [sz, vp]
        L.vce_forward_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.vce_backward_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.vce_forward.argtypes = [i32, i32, i32] + [vp] * 6 + [sz, vp]
        L.vce_backward.argtypes = [i32, i32, i32, i32] + [vp] * 8 + [sz, vp]
        for fn in ("wkv7_forward", "wkv7_backward", "wkv7_backward_noalloc", "wkv7_decode_step", "wkv7_decode_step_fused",
                   "wkv7_gdn_decode_step", "wkv7_gdn_workspace_bytes", "wkv7_gdn_forward",
                   "wkv7_gdn_backward_workspace_bytes", "wkv7_gdn_backward",
                   "wkv7_checkpoint_slots",
                   "wkv7_workspace_bytes", "wkv7_segments_check", "vce_forward_workspace_bytes",
                   "vce_backward_workspace_bytes", "vce_forward", "vce_backward"):
            getattr(L, fn).restype = i32
        _lib = L
    return _lib


def _check(fn, code):
    if code != 0:
        raise WKV7Error(fn, code)


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _cuda(t, name):
    """The first tensor of a call fixes its device, which must be a GPU."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) device tensor")


def _nbytes(t):
    return t.numel() * t.element_size()


def _req(t, name, dev, dtype=None, shape=None):
    """Every tensor a call passes to the library, the caller's own output and
    workspace buffers included: same device, contiguous, and (when given) the
    dtype and shape the C ABI assumes, since it cannot see buffer sizes."""
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Segments:
    """A validated segment table: host copies, device copies (int32) and the
    per-sequence checkpoint slot bases. Build once, reuse across calls."""

    def __init__(self, B, T, seq_start, seq_len, device):
        torch = _torch()
        st = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int32))
        ln = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
        if st.shape != ln.shape or st.ndim != 1 or len(st) == 0:
            raise ValueError("seq_start / seq_len must be equal-length 1-D and non-empty")
        base = np.zeros(len(st), dtype=np.int32)
        slots = ctypes.c_int64(0)
        _check("wkv7_segments_check", lib().wkv7_segments_check(
            B, T, len(st), st.ctypes.data, ln.ctypes.data, base.ctypes.data, ctypes.byref(slots)))
        self.B, self.T = B, T
        self.host_start, self.host_len, self.host_ckpt = st, ln, base
        self.slots = int(slots.value)
        self.num_seqs = len(st)
        self.start = torch.from_numpy(st).to(device)
        self.len = torch.from_numpy(ln).to(device)
        self.ckpt = torch.from_numpy(base).to(device)


def _decay(decay):
    if decay not in DECAY:
        raise ValueError(f"decay must be one of {sorted(DECAY)}")
    return DECAY[decay]


def _desc(B, T, H, dtype, seg: Segments | None, decay="mult", grad_f32=False, n=N):
    d = Desc()
    d.B, d.T, d.H, d.N, d.dtype = B, T, H, n, dtype
    d.decay = _decay(decay)
    d.grad_f32 = 1 if grad_f32 else 0
    if seg is None:
        d.num_seqs = 0
        d.ckpt_slots = 0
    else:
        d.num_seqs = seg.num_seqs
        d.seq_start = seg.start.data_ptr()
        d.seq_len = seg.len.data_ptr()
        d.seq_ckpt = seg.ckpt.data_ptr()
        d.ckpt_slots = seg.slots
    return d


def checkpoint_slots(B, T, seg: Segments | None = None) -> int:
    if seg is not None:
        return seg.slots
    n = ctypes.c_int64(0)
    _check("wkv7_checkpoint_slots", lib().wkv7_checkpoint_slots(B, T, ctypes.byref(n)))
    return int(n.value)


def wkv7_forward(r, w, k, v, a, b, s0=None, *, segments: Segments | None = None,
                 checkpoints: bool = False, state_out: bool = True, y=None, s_out=None,
                 ckpt=None, decay: str = "mult"):
    """y, s_out, ckpt = wkv7_forward(...). s_out/ckpt are None when not requested.
    Head size n = 64 (chunked kernels) or 128 (token-order kernel)."""
    torch = _torch()
    B, T, H, n = r.shape
    dev = r.device
    _cuda(r, "r")
    for name, t in zip("rwkvab", (r, w, k, v, a, b)):
        _req(t, name, dev, r.dtype, r.shape)
    S = segments.num_seqs if segments is not None else B
    if s0 is not None:
        _req(s0, "s0", dev, torch.float32, (S, H, n, n))
    y = torch.empty_like(r) if y is None else y
    _req(y, "y", dev, r.dtype, r.shape)
    if state_out and s_out is None:
        s_out = torch.empty((S, H, n, n), device=dev, dtype=torch.float32)
    if not state_out:
        s_out = None
    if s_out is not None:
        _req(s_out, "s_out", dev, torch.float32, (S, H, n, n))
    slots = checkpoint_slots(B, T, segments)
    if checkpoints and ckpt is None:
        ckpt = torch.empty((slots, H, n, n), device=dev, dtype=torch.float32)
    if not checkpoints:
        ckpt = None
    if ckpt is not None:
        _req(ckpt, "ckpt", dev, torch.float32, (slots, H, n, n))
    d = _desc(B, T, H, _dtype_code(r), segments, decay, n=n)
    _check("wkv7_forward", lib().wkv7_forward(
        ctypes.byref(d), *[_ptr(t) for t in (r, w, k, v, a, b)], _ptr(s0), _ptr(y),
        _ptr(s_out), _ptr(ckpt), _stream()))
    return y, s_out, ckpt


def wkv7_workspace_bytes(B, T, H, dtype, segments: Segments | None = None, n: int = N) -> int:
    d = _desc(B, T, H, dtype, segments, n=n)
    n = ctypes.c_size_t(0)
    _check("wkv7_workspace_bytes", lib().wkv7_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def _backward_args(r, w, k, v, a, b, ckpt, dy, ds_out, segments, want_ds0, grads, grad_f32):
    """Validated outputs (allocated when not given) of a backward call."""
    torch = _torch()
    B, T, H, n = r.shape
    dev = r.device
    _cuda(r, "r")
    for name, t in zip("rwkvab", (r, w, k, v, a, b)):
        _req(t, name, dev, r.dtype, r.shape)
    S = segments.num_seqs if segments is not None else B
    _req(ckpt, "ckpt", dev, torch.float32, (checkpoint_slots(B, T, segments), H, n, n))
    if dy is not None:
        _req(dy, "dy", dev, r.dtype, r.shape)
    if ds_out is not None:
        _req(ds_out, "ds_out", dev, torch.float32, (S, H, n, n))
    names = ("dr", "dw", "dk", "dv", "da", "db")
    gdt = torch.float32 if grad_f32 else r.dtype
    if grads is None:
        grads = {nm: torch.empty(r.shape, device=dev, dtype=gdt) for nm in names}
    for nm in names:
        _req(grads[nm], nm, dev, gdt, r.shape)
    ds0 = torch.empty((S, H, n, n), device=dev, dtype=torch.float32) if want_ds0 else None
    return grads, ds0


def wkv7_backward(r, w, k, v, a, b, ckpt, dy=None, ds_out=None, *,
                  segments: Segments | None = None, want_ds0: bool = True, workspace=None,
                  grads=None, decay: str = "mult", grad_f32: bool = False):
    """Returns dict dr, dw, dk, dv, da, db (dtype of r, or fp32 with grad_f32)
    and ds0 (fp32 or None). With decay="log", dw is the gradient w.r.t. log(decay).
    Head size n = 64 (chunked kernels) or 128 (token-order kernel)."""
    torch = _torch()
    B, T, H, n = r.shape
    grads, ds0 = _backward_args(r, w, k, v, a, b, ckpt, dy, ds_out, segments, want_ds0, grads, grad_f32)
    need = wkv7_workspace_bytes(B, T, H, _dtype_code(r), segments, n=n)
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=r.device, dtype=torch.uint8)
    if workspace is not None:
        _req(workspace, "workspace", r.device)
    ws_bytes = 0 if workspace is None else _nbytes(workspace)
    d = _desc(B, T, H, _dtype_code(r), segments, decay, grad_f32, n=n)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    _check("wkv7_backward", lib().wkv7_backward(
        ctypes.byref(d), *[_ptr(t) for t in (r, w, k, v, a, b)], _ptr(ckpt), _ptr(dy),
        _ptr(ds_out), *[_ptr(grads[nm]) for nm in names], _ptr(ds0), _ptr(workspace),
        ws_bytes, _stream()))
    out = dict(grads)
    out["ds0"] = ds0
    return out


def wkv7_backward_noalloc(r, w, k, v, a, b, ckpt, dy=None, ds_out=None, *,
                          segments: Segments | None = None, want_ds0: bool = True, grads=None,
                          ds0=None, decay: str = "mult", grad_f32: bool = False):
    """wkv7_backward with the library's static per-device scratch instead of a
    workspace (the C call allocates nothing; pass grads and ds0 to allocate
    nothing here either). Returns the same dict as wkv7_backward."""
    torch = _torch()
    B, T, H, n = r.shape
    if ds0 is not None:
        want_ds0 = False
    grads, ds0_new = _backward_args(r, w, k, v, a, b, ckpt, dy, ds_out, segments, want_ds0, grads,
                                    grad_f32)
    if ds0 is None:
        ds0 = ds0_new
    else:
        S = segments.num_seqs if segments is not None else B
        _req(ds0, "ds0", r.device, torch.float32, (S, H, n, n))
    d = _desc(B, T, H, _dtype_code(r), segments, decay, grad_f32, n=n)
    names = ("dr", "dw", "dk", "dv", "da", "db")
    _check("wkv7_backward_noalloc", lib().wkv7_backward_noalloc(
        ctypes.byref(d), *[_ptr(t) for t in (r, w, k, v, a, b)], _ptr(ckpt), _ptr(dy),
        _ptr(ds_out), *[_ptr(grads[nm]) for nm in names], _ptr(ds0), _stream()))
    out = dict(grads)
    out["ds0"] = ds0
    return out


STATIC_SCRATCH_BYTES = 128 << 20


def wkv7_decode_step(r, w, k, v, a, b, s_in, s_out=None, y=None, *, decay: str = "mult"):
    """One token per (sequence, head): streams [B, H, n], state [B, H, n, n]
    with head size n = 64 or 128. Pass s_out=s_in to update the state in
    place. Returns (y, s_out)."""
    torch = _torch()
    B, H, n = r.shape
    dev = r.device
    _cuda(r, "r")
    for name, t in zip("rwkvab", (r, w, k, v, a, b)):
        _req(t, name, dev, r.dtype, r.shape)
    _req(s_in, "s_in", dev, torch.float32, (B, H, n, n))
    if s_out is None:
        s_out = torch.empty_like(s_in)
    _req(s_out, "s_out", dev, torch.float32, (B, H, n, n))
    y = torch.empty_like(r) if y is None else y
    _req(y, "y", dev, r.dtype, r.shape)
    _check("wkv7_decode_step", lib().wkv7_decode_step(
        B, H, n, _dtype_code(r), _decay(decay), *[_ptr(t) for t in (r, w, k, v, a, b)], _ptr(s_in),
        _ptr(s_out), _ptr(y), _stream()))
    return y, s_out


def wkv7_decode_step_fused(r, w, k, v, a, b, s_in, g, ln_w, ln_b, r_k, eps, s_out=None, out=None,
                           y=None, *, want_y: bool = False, decay: str = "mult"):
    """One decode step with the per-head output epilogue:
    out = (GroupNorm_h(y) * ln_w + ln_b + (sum_j r_j k_j r_k[h, j]) v) * g.
    Streams and g [B, H, 64] (one dtype); ln_w, ln_b, r_k [H, 64] fp32; state
    [B, H, 64, 64] fp32 (s_out=s_in updates it in place). Returns
    (out, s_out, y), y None unless want_y or given."""
    torch = _torch()
    B, H, n = r.shape
    dev = r.device
    _cuda(r, "r")
    for name, t in zip("rwkvab", (r, w, k, v, a, b)):
        _req(t, name, dev, r.dtype, r.shape)
    _req(g, "g", dev, r.dtype, r.shape)
    for name, t in (("ln_w", ln_w), ("ln_b", ln_b), ("r_k", r_k)):
        _req(t, name, dev, torch.float32, (H, N))
    _req(s_in, "s_in", dev, torch.float32, (B, H, N, N))
    if s_out is None:
        s_out = torch.empty_like(s_in)
    _req(s_out, "s_out", dev, torch.float32, (B, H, N, N))
    out = torch.empty_like(r) if out is None else out
    _req(out, "out", dev, r.dtype, r.shape)
    if y is None and want_y:
        y = torch.empty_like(r)
    if y is not None:
        _req(y, "y", dev, r.dtype, r.shape)
    _check("wkv7_decode_step_fused", lib().wkv7_decode_step_fused(
        B, H, n, _dtype_code(r), _decay(decay), *[_ptr(t) for t in (r, w, k, v, a, b)], _ptr(s_in),
        _ptr(s_out), _ptr(g), _ptr(ln_w), _ptr(ln_b), _ptr(r_k), float(eps), _ptr(out), _ptr(y),
        _stream()))
    return out, s_out, y


def wkv7_gdn_decode_step(q, k, v, g, beta, s_in, s_out=None, out=None):
    """One token of a gated DeltaNet layer through the RWKV-7 remap: q, k
    [B, Hk, N], v [B, H, N] (one dtype), g, beta fp32 [B, H], state fp32
    [B, H, N, N] (N = 64 or 128). s_out=s_in updates in place. Returns
    (out [B, H, N], s_out)."""
    torch = _torch()
    dev = v.device
    _cuda(v, "v")
    B, H, N = v.shape
    Hk = q.shape[1]
    dt = v.dtype
    _req(q, "q", dev, dt, (B, Hk, N))
    _req(k, "k", dev, dt, (B, Hk, N))
    _req(v, "v", dev, dt)
    _req(g, "g", dev, torch.float32, (B, H))
    _req(beta, "beta", dev, torch.float32, (B, H))
    _req(s_in, "s_in", dev, torch.float32, (B, H, N, N))
    s_out = torch.empty_like(s_in) if s_out is None else s_out
    _req(s_out, "s_out", dev, torch.float32, (B, H, N, N))
    out = torch.empty_like(v) if out is None else out
    _req(out, "out", dev, dt, (B, H, N))
    _check("wkv7_gdn_decode_step", lib().wkv7_gdn_decode_step(
        B, H, Hk, N, _dtype_code(v), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(s_in), _ptr(s_out), _ptr(out), _stream()))
    return out, s_out


def wkv7_gdn_workspace_bytes(B, T, Hk, N) -> int:
    out = ctypes.c_size_t(0)
    _check("wkv7_gdn_workspace_bytes", lib().wkv7_gdn_workspace_bytes(B, T, Hk, N, ctypes.byref(out)))
    return out.value


def wkv7_gdn_forward(q, k, v, g, beta, s0=None, *, out=None, want_state=True, workspace=None):
    """A dense batch of gated DeltaNet tokens through the RWKV-7 remap: q, k
    [B, T, Hk, N], v [B, T, H, N] (one dtype), g, beta fp32 [B, T, H], s0
    fp32 [B, H, N, N] or None. Returns (out [B, T, H, N], s_out or None)."""
    torch = _torch()
    dev = v.device
    _cuda(v, "v")
    B, T, H, N = v.shape
    Hk = q.shape[2]
    dt = v.dtype
    _req(q, "q", dev, dt, (B, T, Hk, N))
    _req(k, "k", dev, dt, (B, T, Hk, N))
    _req(v, "v", dev, dt)
    _req(g, "g", dev, torch.float32, (B, T, H))
    _req(beta, "beta", dev, torch.float32, (B, T, H))
    if s0 is not None:
        _req(s0, "s0", dev, torch.float32, (B, H, N, N))
    out = torch.empty_like(v) if out is None else out
    _req(out, "out", dev, dt, (B, T, H, N))
    s_out = torch.empty((B, H, N, N), device=dev, dtype=torch.float32) if want_state else None
    need = wkv7_gdn_workspace_bytes(B, T, Hk, N)
    ws = torch.empty(need, device=dev, dtype=torch.uint8) if workspace is None else workspace
    _req(ws, "workspace", dev)
    _check("wkv7_gdn_forward", lib().wkv7_gdn_forward(
        B, T, H, Hk, N, _dtype_code(v), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        _ptr(out), _ptr(s_out), _ptr(ws), _nbytes(ws), _stream()))
    return out, s_out


def wkv7_gdn_backward_workspace_bytes(B, T, H, Hk, N) -> int:
    out = ctypes.c_size_t(0)
    _check("wkv7_gdn_backward_workspace_bytes",
           lib().wkv7_gdn_backward_workspace_bytes(B, T, H, Hk, N, ctypes.byref(out)))
    return int(out.value)


def wkv7_gdn_backward(q, k, v, g, beta, s0=None, dout=None, ds_out=None, *, want_ds0=True, workspace=None):
    """Gradients of sum <dout, out> + <ds_out, S_T> for wkv7_gdn_forward.
    Returns dict dq, dk ([B, T, Hk, N]), dv ([B, T, H, N]) in the inputs'
    dtype, dg, dbeta (fp32 [B, T, H]) and ds0 (fp32 [B, H, N, N] or None)."""
    torch = _torch()
    dev = v.device
    _cuda(v, "v")
    B, T, H, N = v.shape
    Hk = q.shape[2]
    dt = v.dtype
    _req(q, "q", dev, dt, (B, T, Hk, N))
    _req(k, "k", dev, dt, (B, T, Hk, N))
    _req(v, "v", dev, dt)
    _req(g, "g", dev, torch.float32, (B, T, H))
    _req(beta, "beta", dev, torch.float32, (B, T, H))
    if s0 is not None:
        _req(s0, "s0", dev, torch.float32, (B, H, N, N))
    if dout is not None:
        _req(dout, "dout", dev, dt, (B, T, H, N))
    if ds_out is not None:
        _req(ds_out, "ds_out", dev, torch.float32, (B, H, N, N))
    res = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
           "ds0": torch.empty((B, H, N, N), device=dev, dtype=torch.float32) if want_ds0 else None}
    need = wkv7_gdn_backward_workspace_bytes(B, T, H, Hk, N)
    ws = torch.empty(need, device=dev, dtype=torch.uint8) if workspace is None else workspace
    _req(ws, "workspace", dev)
    _check("wkv7_gdn_backward", lib().wkv7_gdn_backward(
        B, T, H, Hk, N, _dtype_code(v), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        _ptr(dout), _ptr(ds_out), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]),
        _ptr(res["dbeta"]), _ptr(res["ds0"]), _ptr(ws), _nbytes(ws), _stream()))
    return res


def wkv7_abi_version() -> int:
    return int(lib().wkv7_abi_version())


def wkv7_status_string(code: int) -> str:
    return lib().wkv7_status_string(code).decode()


def wkv7_segments_check(B, T, seq_start, seq_len):
    """Host validation of a segment table; returns (seq_ckpt, slots)."""
    st = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int32))
    ln = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int32))
    base = np.zeros(len(st), dtype=np.int32)
    slots = ctypes.c_int64(0)
    _check("wkv7_segments_check", lib().wkv7_segments_check(
        B, T, len(st), st.ctypes.data if len(st) else None, ln.ctypes.data if len(ln) else None,
        base.ctypes.data if len(st) else None, ctypes.byref(slots)))
    return base, int(slots.value)


def wkv7_checkpoint_slots(B, T) -> int:
    return checkpoint_slots(B, T)
