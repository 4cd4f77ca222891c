"""C-ABI checks that need no GPU: the library loads, exports every function
include/wkv7.h declares, and rejects bad arguments with the documented status
codes before touching the HIP runtime (no compute call is made here)."""
import ctypes

import numpy as np
import pytest

from linear_recurrent_lm_amd import wkv7 as W
from linear_recurrent_lm_amd import synth

INVALID, UNSUPPORTED, WS = 1, 2, 3

# Fake, 16-byte aligned, non-null device addresses: validation must fail on
# another argument before any of these could be dereferenced.
P = [ctypes.c_void_p(0x1000 * (q + 1)) for q in range(20)]


def desc(**kw):
    d = W.Desc()
    d.B, d.T, d.H, d.N, d.dtype, d.num_seqs, d.ckpt_slots = 2, 32, 4, 64, 1, 0, 0
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def fwd(d, *, ptrs=None, s0=None, y=P[6], s_out=None, ckpt=None):
    ptrs = ptrs or P[:6]
    return W.lib().wkv7_forward(ctypes.byref(d) if d is not None else None, *ptrs, s0, y,
                                s_out, ckpt, None)


def test_library_exports_every_declared_function():
    L = W.lib()
    names = W.declared_functions()
    assert {"wkv7_forward", "wkv7_backward", "wkv7_decode_step"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_version_and_status_strings():
    assert W.wkv7_abi_version() == 2
    assert W.wkv7_status_string(0) == "ok"
    assert W.wkv7_status_string(3) == "workspace too small"
    assert W.wkv7_status_string(99) == "unknown status"


def test_forward_rejects_bad_descriptors():
    assert fwd(None) == INVALID
    assert fwd(desc(N=96)) == UNSUPPORTED
    assert fwd(desc(N=256)) == UNSUPPORTED
    # head size 128 is a forward size: with N = 128 the other checks still apply
    assert fwd(desc(N=128, B=0)) == INVALID
    assert fwd(desc(N=128, dtype=7)) == UNSUPPORTED
    assert fwd(desc(dtype=7)) == UNSUPPORTED
    assert fwd(desc(dtype=-1)) == UNSUPPORTED
    assert fwd(desc(decay=2)) == UNSUPPORTED                    # neither multiplicative nor log
    assert fwd(desc(grad_f32=3)) == INVALID
    for bad in (dict(B=0), dict(T=0), dict(H=0), dict(H=65537), dict(T=-5), dict(num_seqs=-1)):
        assert fwd(desc(**bad)) == INVALID, bad
    assert fwd(desc(B=1 << 20, T=1 << 12)) == INVALID          # B*T over int32
    assert fwd(desc(num_seqs=3)) == INVALID                     # tables missing


def test_forward_rejects_bad_pointers():
    d = desc()
    for q in range(6):
        ptrs = list(P[:6]); ptrs[q] = None
        assert fwd(d, ptrs=ptrs) == INVALID
        ptrs = list(P[:6]); ptrs[q] = ctypes.c_void_p(0x1004)
        assert fwd(d, ptrs=ptrs) == INVALID
    assert fwd(d, y=None) == INVALID
    assert fwd(d, s0=ctypes.c_void_p(0x2008)) == INVALID
    # s_out may not alias s0
    assert fwd(d, s0=P[10], s_out=ctypes.c_void_p(P[10].value + 4096)) == INVALID
    # segment-mode checkpoints need the slot table
    arr = ctypes.c_void_p(0x9000)
    assert fwd(desc(num_seqs=2, seq_start=arr.value, seq_len=arr.value), ckpt=P[12]) == INVALID


def test_backward_rejects_bad_arguments():
    L = W.lib()
    d = desc()
    grads = P[7:13]
    call = lambda d, ckpt=P[6], grads=grads, ws=None, wsb=0: L.wkv7_backward(
        ctypes.byref(d), *P[:6], ckpt, None, None, *grads, None, ws, wsb, None)
    assert call(desc(N=32)) == UNSUPPORTED
    assert call(desc(N=96)) == UNSUPPORTED
    # head size 128 takes no workspace; its other checks still apply
    assert W.wkv7_workspace_bytes(2, 32, 4, 1, n=128) == 0
    assert call(desc(N=128), ckpt=None) == INVALID
    assert call(desc(N=128, dtype=7)) == UNSUPPORTED
    assert call(d, ckpt=None) == INVALID
    for q in range(6):
        g = list(grads); g[q] = None
        assert call(d, grads=g) == INVALID


def test_decode_rejects_bad_arguments():
    L = W.lib()
    call = lambda B=4, H=2, N=64, dt=1, dc=0, s_in=P[7], s_out=P[8], y=P[6]: L.wkv7_decode_step(
        B, H, N, dt, dc, *P[:6], s_in, s_out, y, None)
    assert call(N=32) == UNSUPPORTED
    assert call(N=96) == UNSUPPORTED
    assert call(N=256) == UNSUPPORTED
    assert call(dt=3) == UNSUPPORTED
    assert call(dc=5) == UNSUPPORTED
    assert call(B=0) == INVALID
    assert call(s_in=None) == INVALID
    assert call(y=None) == INVALID
    assert call(N=128, y=None) == INVALID      # head size 128 passes the size check, then fails here
    # overlapping but not identical state buffers
    assert call(s_in=P[7], s_out=ctypes.c_void_p(P[7].value + 16)) == INVALID


def test_fused_decode_rejects_bad_arguments():
    L = W.lib()

    def call(B=4, H=2, N=64, dt=1, dc=0, g=P[9], ln_w=P[10], ln_b=P[11], r_k=P[12], eps=1e-5,
             out=P[13], y=None, s_in=P[7], s_out=P[8]):
        return L.wkv7_decode_step_fused(B, H, N, dt, dc, *P[:6], s_in, s_out, g, ln_w, ln_b, r_k,
                                        eps, out, y, None)
    assert call(N=32) == UNSUPPORTED
    assert call(N=128) == UNSUPPORTED          # the fused epilogue is built for head size 64
    assert call(dt=3) == UNSUPPORTED
    assert call(dc=5) == UNSUPPORTED
    assert call(B=0) == INVALID
    assert call(out=None) == INVALID
    for name in ("g", "ln_w", "ln_b", "r_k"):
        assert call(**{name: None}) == INVALID, name
        assert call(**{name: ctypes.c_void_p(0x1004)}) == INVALID, name
    assert call(y=ctypes.c_void_p(0x1008)) == INVALID            # y is optional but aligned
    for eps in (-1e-5, float("nan"), float("inf")):
        assert call(eps=eps) == INVALID, eps
    assert call(s_in=P[7], s_out=ctypes.c_void_p(P[7].value + 16)) == INVALID


def test_gdn_decode_rejects_bad_arguments():
    L = W.lib()

    def call(B=4, H=4, Hk=2, N=128, dt=1, q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4],
             s_in=P[5], s_out=P[6], out=P[7]):
        return L.wkv7_gdn_decode_step(B, H, Hk, N, dt, q, k, v, g, beta, s_in, s_out, out, None)
    assert call(N=96) == UNSUPPORTED
    assert call(N=256) == UNSUPPORTED
    assert call(dt=3) == UNSUPPORTED
    assert call(B=0) == INVALID
    assert call(Hk=0) == INVALID
    assert call(H=6, Hk=4) == INVALID                      # key heads must divide value heads
    for name in ("q", "k", "v", "g", "beta", "s_in", "s_out", "out"):
        assert call(**{name: None}) == INVALID, name
    assert call(q=ctypes.c_void_p(P[0].value + 8)) == INVALID
    assert call(g=ctypes.c_void_p(P[3].value + 2)) == INVALID
    far = [ctypes.c_void_p((q + 1) << 40) for q in range(8)]
    # partial overlap of the states, and out inside s_out
    assert call(s_in=far[5], s_out=ctypes.c_void_p(far[5].value + 16), q=far[0], k=far[1],
                v=far[2], g=far[3], beta=far[4], out=far[7]) == INVALID
    assert call(s_in=far[5], s_out=far[6], out=ctypes.c_void_p(far[6].value + 64), q=far[0],
                k=far[1], v=far[2], g=far[3], beta=far[4]) == INVALID


def test_gdn_forward_rejects_bad_arguments():
    L = W.lib()
    far = [ctypes.c_void_p((q + 1) << 40) for q in range(12)]
    BIG = 1 << 38

    def call(B=2, T=8, H=4, Hk=2, N=128, dt=1, q=far[0], k=far[1], v=far[2], g=far[3],
             beta=far[4], s0=None, out=far[5], s_out=far[6], ws=far[7], nbytes=BIG):
        return L.wkv7_gdn_forward(B, T, H, Hk, N, dt, q, k, v, g, beta, s0, out, s_out, ws,
                                  nbytes, None)
    assert call(N=96) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(T=0) == INVALID
    assert call(H=6, Hk=4) == INVALID
    for name in ("q", "k", "v", "g", "beta", "out", "ws"):
        assert call(**{name: None}) == INVALID, name
    assert call(q=ctypes.c_void_p(far[0].value + 8)) == INVALID
    assert call(s0=ctypes.c_void_p(far[8].value + 4)) == INVALID
    assert call(out=ctypes.c_void_p(far[2].value + 64)) == INVALID       # out overlaps v
    assert call(s_out=ctypes.c_void_p(far[7].value + 256)) == INVALID    # s_out overlaps the workspace
    need = W.wkv7_gdn_workspace_bytes(2, 8, 2, 128)
    assert need == 2 * 2 * 8 * 2 * 128 * 4
    assert call(nbytes=need - 1) == WS
    with pytest.raises(W.WKV7Error):
        W.wkv7_gdn_workspace_bytes(2, 8, 2, 96)


def test_gdn_backward_rejects_bad_arguments():
    L = W.lib()
    far = [ctypes.c_void_p((q + 1) << 40) for q in range(16)]
    BIG = 1 << 38

    def call(B=2, T=8, H=4, Hk=2, N=128, dt=1, q=far[0], k=far[1], v=far[2], g=far[3], beta=far[4],
             s0=None, dout=far[5], ds_out=None, dq=far[6], dk=far[7], dv=far[8], dg=far[9], dbeta=far[10],
             ds0=far[11], ws=far[12], nbytes=BIG):
        return L.wkv7_gdn_backward(B, T, H, Hk, N, dt, q, k, v, g, beta, s0, dout, ds_out, dq, dk, dv, dg,
                                   dbeta, ds0, ws, nbytes, None)
    assert call(N=96) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(T=0) == INVALID
    assert call(H=6, Hk=4) == INVALID
    for name in ("q", "k", "v", "g", "beta", "dq", "dk", "dv", "dg", "dbeta", "ws"):
        assert call(**{name: None}) == INVALID, name
    assert call(dout=ctypes.c_void_p(far[5].value + 8)) == INVALID          # misaligned
    assert call(ds0=ctypes.c_void_p(far[11].value + 4)) == INVALID
    assert call(dv=ctypes.c_void_p(far[2].value + 64)) == INVALID           # dv overlaps v
    assert call(dg=ctypes.c_void_p(far[12].value + 256)) == INVALID         # dg overlaps the workspace
    assert call(dq=far[7]) == INVALID                                      # dq is dk
    need = W.wkv7_gdn_backward_workspace_bytes(2, 8, 4, 2, 128)
    key, val = 2 * 8 * 2 * 128 * 4, 2 * 8 * 4 * 128 * 4
    assert need == 2 * key + 13 * val + 2 * 4 * 128 * 128 * 4              # + checkpoints; no WKV-7 workspace
    assert W.wkv7_gdn_backward_workspace_bytes(2, 8, 4, 2, 64) > 0
    assert call(nbytes=need - 1) == WS
    with pytest.raises(W.WKV7Error):
        W.wkv7_gdn_backward_workspace_bytes(2, 8, 4, 2, 96)


def test_checkpoint_slots():
    assert W.checkpoint_slots(3, 33) == 9
    assert W.checkpoint_slots(2, 16) == 2
    assert W.checkpoint_slots(1, 1) == 1
    n = ctypes.c_int64()
    assert W.lib().wkv7_checkpoint_slots(0, 5, ctypes.byref(n)) == INVALID


def test_workspace_query():
    # per checkpoint slot and head: an fp32 64x64 state gradient, a 16x64 drhs, a 16x16 W
    per = 64 * 64 + 16 * 64 + 16 * 16
    assert W.wkv7_workspace_bytes(4, 64, 8, 1) == 4 * 4 * 8 * per * 4
    assert W.wkv7_workspace_bytes(3, 33, 2, 0) == 9 * 2 * per * 4
    # segment mode adds the work-item list: a count and ceil(slots / 8) + num_seqs pairs, 256-aligned
    n = ctypes.c_size_t()
    d = desc(num_seqs=3, seq_start=0x9000, seq_len=0x9000, ckpt_slots=9, H=2)
    assert W.lib().wkv7_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 9 * 2 * per * 4 + 256
    assert W.lib().wkv7_workspace_bytes(ctypes.byref(desc(N=48)), ctypes.byref(n)) == UNSUPPORTED
    # head size 128: none (one workgroup per unit sums every gradient)
    n.value = 123
    assert W.lib().wkv7_workspace_bytes(ctypes.byref(desc(N=128)), ctypes.byref(n)) == 0
    assert n.value == 0


def test_segments_check_matches_layout_helpers():
    lengths = synth.ragged_lengths(64, 16, 2048, seed=4)
    T_pad, st, ln = synth.packed_layout(lengths, 4)
    order, st_s, ln_s = synth.sorted_table(st, ln)
    base, slots = W.wkv7_segments_check(4, T_pad, st_s, ln_s)
    ref_base, ref_slots = synth.checkpoint_bases(ln_s)
    assert slots == ref_slots and np.array_equal(base, ref_base)
    assert slots == synth.checkpoint_bases(lengths)[1]
    st2, ln2 = synth.padded_layout(lengths, 2048)
    base2, slots2 = W.wkv7_segments_check(64, 2048, st2, ln2)
    assert np.array_equal(base2, synth.checkpoint_bases(lengths)[0])
    # the packed table in sequence order is not sorted by start: rejected
    with pytest.raises(W.WKV7Error):
        W.wkv7_segments_check(4, T_pad, st, ln)


@pytest.mark.parametrize("start,length", [
    ([0, 10], [12, 4]),        # overlap
    ([10, 0], [4, 4]),         # unsorted
    ([30], [5]),               # crosses a row boundary (T=32)
    ([0], [-1]),               # negative length
    ([60], [10]),              # past the end (B*T = 64)
])
def test_segments_check_rejects(start, length):
    with pytest.raises(W.WKV7Error) as e:
        W.wkv7_segments_check(2, 32, start, length)
    assert e.value.code == INVALID


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(W, "_lib", None)
    monkeypatch.setattr(W, "LIB_PATH", "/nonexistent/libwkv7.so")
    with pytest.raises(RuntimeError, match="missing"):
        W.lib()


# Fake device addresses 2^40 bytes apart: no two buffers of the small shapes
# below overlap unless a test places one inside another on purpose. Every call
# here is expected to fail validation (with no GPU, a call that passed it would
# return the HIP error instead, failing the test).
FAR = [ctypes.c_void_p((q + 1) << 40) for q in range(24)]


def inside(p, off=64):
    return ctypes.c_void_p(p.value + off)


def test_forward_rejects_overlapping_outputs():
    d = desc()                          # B=2, T=32, H=4, bf16: 32 KiB streams
    L = W.lib()
    base = dict(ptrs=FAR[:6], s0=FAR[6], y=FAR[7], s_out=FAR[8], ckpt=FAR[9])

    def call(**kw):
        a = dict(base, **kw)
        return L.wkv7_forward(ctypes.byref(d), *a["ptrs"], a["s0"], a["y"], a["s_out"], a["ckpt"], None)
    for q in range(6):                                  # y over each input stream
        assert call(y=inside(FAR[q])) == INVALID, q
    assert call(y=inside(FAR[6])) == INVALID            # y over s0
    assert call(s_out=inside(FAR[3])) == INVALID        # s_out over v
    assert call(s_out=inside(FAR[6])) == INVALID        # s_out over s0
    assert call(ckpt=inside(FAR[0])) == INVALID         # checkpoints over r
    assert call(ckpt=inside(FAR[7])) == INVALID         # checkpoints over y
    assert call(y=inside(FAR[8])) == INVALID            # y over s_out


def test_backward_rejects_overlapping_outputs():
    d = desc()
    L = W.lib()
    need = W.wkv7_workspace_bytes(2, 32, 4, 1)
    base = dict(ins=FAR[:6], ckpt=FAR[6], dy=FAR[7], ds_out=FAR[8], grads=FAR[9:15], ds0=FAR[15],
                ws=FAR[16])

    def call(**kw):
        a = dict(base, **kw)
        return L.wkv7_backward(ctypes.byref(d), *a["ins"], a["ckpt"], a["dy"], a["ds_out"], *a["grads"],
                               a["ds0"], a["ws"], need, None)
    for q in range(6):
        g = list(FAR[9:15]); g[q] = inside(FAR[q])      # gradient over its own input
        assert call(grads=g) == INVALID, q
    g = list(FAR[9:15]); g[2] = inside(FAR[9])          # two gradients sharing bytes
    assert call(grads=g) == INVALID
    assert call(ds0=inside(FAR[6])) == INVALID          # ds0 over the checkpoints
    assert call(ws=inside(FAR[7])) == INVALID           # workspace over dy
    assert call(ws=inside(FAR[9])) == INVALID           # workspace over dr
    assert call(ds0=inside(FAR[8])) == INVALID          # ds0 over ds_out


def test_decode_rejects_overlapping_outputs():
    L = W.lib()

    def call(y=FAR[6], s_in=FAR[7], s_out=FAR[8], ins=None):
        return L.wkv7_decode_step(4, 2, 64, 1, 0, *(ins or FAR[:6]), s_in, s_out, y, None)
    for q in range(6):                 # y over r..b (the kernel reads r while writing y)
        assert call(y=inside(FAR[q], 16)) == INVALID, q
    assert call(y=inside(FAR[7])) == INVALID            # y over s_in
    assert call(y=inside(FAR[7]), s_out=FAR[7]) == INVALID   # y over the in-place state
    ins = list(FAR[:6]); ins[4] = inside(FAR[8])        # s_out over an input
    assert call(ins=ins) == INVALID

    def fused(out=FAR[13], y=None, g=FAR[9], ln_w=FAR[10]):
        return L.wkv7_decode_step_fused(4, 2, 64, 1, 0, *FAR[:6], FAR[7], FAR[8], g, ln_w, FAR[11],
                                        FAR[12], 1e-5, out, y, None)
    assert fused(out=inside(FAR[0], 16)) == INVALID     # out over r
    assert fused(out=inside(FAR[9])) == INVALID         # out over the gate
    assert fused(y=inside(FAR[13])) == INVALID          # y over out
    assert fused(ln_w=inside(FAR[8])) == INVALID        # a parameter inside s_out


def test_gdn_decode_rejects_overlapping_outputs():
    L = W.lib()

    def call(out=FAR[7], s_in=FAR[5], s_out=FAR[6], q=FAR[0], v=FAR[2]):
        return L.wkv7_gdn_decode_step(4, 4, 2, 128, 1, q, FAR[1], v, FAR[3], FAR[4], s_in, s_out, out, None)
    assert call(out=inside(FAR[2])) == INVALID          # out over v
    assert call(out=inside(FAR[5])) == INVALID          # out over s_in (out of place)
    assert call(out=inside(FAR[5]), s_out=FAR[5]) == INVALID  # out over the in-place state
    assert call(q=inside(FAR[6])) == INVALID            # s_out over q


def test_backward_noalloc_size_limit_and_checks():
    """The static-scratch backward refuses descriptors whose per-chunk results
    exceed WKV7_STATIC_SCRATCH_BYTES, and validates like wkv7_backward."""
    L = W.lib()
    big = desc(B=4, T=4096, H=32)
    assert W.wkv7_workspace_bytes(4, 4096, 32, 1) > W.STATIC_SCRATCH_BYTES

    def call(d, ckpt=FAR[6], grads=None, dr=None):
        g = list(grads or FAR[9:15])
        return L.wkv7_backward_noalloc(ctypes.byref(d), *FAR[:6], ckpt, None, None, *g, None, None)
    assert call(big) == WS
    assert call(desc(N=128)) == UNSUPPORTED
    assert call(desc(), ckpt=None) == INVALID
    g = list(FAR[9:15]); g[1] = inside(FAR[1])
    assert call(desc(), grads=g) == INVALID
    # the header's limit and the binding's agree
    text = open(W.HEADER).read()
    assert "#define WKV7_STATIC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert W.STATIC_SCRATCH_BYTES == 128 << 20
