"""Seeded synthetic inputs for the WKV-7 recurrence.

This module only draws random numbers and shapes them into the input streams
(r, w, k, v, a, b), initial states, upstream gradients and segment tables.
It holds none of the recurrence's arithmetic and is the one piece shared by
the CPU oracle side (tests, CPU baseline) and the GPU side (binding tests,
benchmark), so that both read bit-identical inputs.

Distributions (the configuration recipe used throughout):
  r, k, v ~ N(0, 1)
  w = exp(-exp(x)),  x ~ U(-6, -0.5)       -> w in [0.5452, 0.9975]
  kk = k / ||k||_2 over the head dimension, computed from the fp32 k
  a = -kk,  b = kk * sigmoid(z),  z ~ N(0, 1)
  optional initial state ~ N(0, std^2), upstream dy ~ N(0, 1)
With decay="log" the w stream instead holds -exp(x), the logarithm of the same
decay (the kernels then take exp of it).
Values are produced in fp32 and, for bf16 / fp16 workloads, rounded to that
type with round-to-nearest-even; the fp32 arrays returned then hold exactly
the rounded values, so upcasting them to fp64 is exact.

Arrays use the [B, T, H, N] layout (N contiguous); states are [S, H, N, N]
with the row index = value index and the column index = key index.
"""
from __future__ import annotations

import dataclasses
import numpy as np

CHUNK = 16


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = (((u + bias) >> 16) << 16).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def round_f16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest fp16 (ties to even); returns fp32."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of an 'f32', 'bf16' or 'f16' stream, held in fp32."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return round_f16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


DTYPES = ("f32", "bf16", "f16")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Inputs:
    """One batch of WKV-7 inputs. Float arrays are fp32 holding the exact
    values the kernels read (rounded to dtype when it is 'bf16' or 'f16');
    w holds log(decay) when decay == 'log'."""
    dtype: str
    r: np.ndarray
    w: np.ndarray
    k: np.ndarray
    v: np.ndarray
    a: np.ndarray
    b: np.ndarray
    s0: np.ndarray | None = None
    dy: np.ndarray | None = None
    ds_out: np.ndarray | None = None
    seq_start: np.ndarray | None = None   # int32, flat token index b*T + t
    seq_len: np.ndarray | None = None     # int32
    decay: str = "mult"

    @property
    def shape(self):
        return self.r.shape

    def streams(self):
        return (self.r, self.w, self.k, self.v, self.a, self.b)


def _draw_streams(rng, shape, decay="mult"):
    r = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    x = (np.float32(-6.0) + np.float32(5.5) * rng.random(shape, dtype=np.float32))
    z = rng.standard_normal(shape, dtype=np.float32)
    w = -np.exp(x) if decay == "log" else np.exp(-np.exp(x))
    nrm = np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=-1, keepdims=True))
    kk = (k / np.maximum(nrm, 1e-30)).astype(np.float32)
    a = -kk
    b = (kk * (1.0 / (1.0 + np.exp(-z)))).astype(np.float32)
    return [np.ascontiguousarray(t, dtype=np.float32) for t in (r, w, k, v, a, b)]


def make_inputs(B: int, T: int, H: int, N: int = 64, *, seed: int = 0,
                dtype: str = "bf16", s0_std: float = 0.0, with_dy: bool = False,
                ds_out_std: float = 0.0, decay: str = "mult") -> Inputs:
    """Dense batch: B rows of T tokens, H heads of size N."""
    if dtype not in DTYPES:
        raise ValueError(dtype)
    if decay not in ("mult", "log"):
        raise ValueError(decay)
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, T, H, N)
    streams = [round_to(s, dtype) for s in _draw_streams(rng, shape, decay)]
    s0 = None
    if s0_std > 0:
        s0 = (rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(s0_std))
    dy = None
    if with_dy:
        dy = round_to(rng.standard_normal(shape, dtype=np.float32), dtype)
    ds_out = None
    if ds_out_std > 0:
        ds_out = rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(ds_out_std)
    return Inputs(dtype, *streams, s0=s0, dy=dy, ds_out=ds_out, decay=decay)


def ragged_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths drawn uniformly from the integers lo..hi inclusive."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)


def packed_layout(lengths: np.ndarray, streams: int):
    """Assign sequence i to stream i mod `streams`, concatenated in order of i.
    Each stream is right-padded to a multiple of CHUNK tokens.
    Returns (T_pad, seq_start, seq_len) with seq_start a flat index b*T_pad + t."""
    lengths = np.asarray(lengths, dtype=np.int64)
    fill = np.zeros(streams, dtype=np.int64)
    pos = np.zeros(len(lengths), dtype=np.int64)
    row = np.zeros(len(lengths), dtype=np.int64)
    for i, L in enumerate(lengths):
        s = i % streams
        row[i] = s
        pos[i] = fill[s]
        fill[s] += L
    T_pad = int(CHUNK * -(-max(int(fill.max()), 1) // CHUNK))
    start = row * T_pad + pos
    return T_pad, start.astype(np.int32), lengths.astype(np.int32)


def sorted_table(seq_start, seq_len):
    """Order a segment table by start token (the library requires sorted
    starts). Returns (order, start[order], len[order]); entry q of the sorted
    table is sequence order[q] of the original table."""
    seq_start = np.asarray(seq_start, dtype=np.int64)
    order = np.argsort(seq_start, kind="stable")
    return (order, seq_start[order].astype(np.int32),
            np.asarray(seq_len)[order].astype(np.int32))


def padded_layout(lengths: np.ndarray, T: int):
    """Right-padded layout: sequence i occupies row i from token 0."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.max(initial=0) > T:
        raise ValueError("sequence longer than the row")
    start = np.arange(len(lengths), dtype=np.int64) * T
    return start.astype(np.int32), lengths.astype(np.int32)


def make_segment_inputs(lengths: np.ndarray, H: int, N: int = 64, *, seed: int = 4,
                        dtype: str = "bf16", s0_std: float = 0.0, with_dy: bool = False):
    """Draw the tokens of `len(lengths)` sequences once, as one flat
    [sum(lengths), H, N] array per stream (sequence i's tokens are contiguous,
    in order of i), plus optional per-sequence states and dy.
    Use `scatter_segments` to place them into a packed or padded layout."""
    total = int(np.sum(lengths))
    base = make_inputs(1, total, H, N, seed=seed, dtype=dtype, s0_std=0.0, with_dy=with_dy)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    s0 = None
    if s0_std > 0:
        s0 = rng.standard_normal((len(lengths), H, N, N), dtype=np.float32) * np.float32(s0_std)
    flat = {name: getattr(base, name)[0] for name in ("r", "w", "k", "v", "a", "b")}
    if with_dy:
        flat["dy"] = base.dy[0]
    return flat, s0


def scatter_segments(flat: dict, lengths, seq_start, B: int, T: int, *,
                     fill: float = float("nan"), dtype: str = "bf16") -> Inputs:
    """Place per-sequence tokens into a [B, T, H, N] layout at the given flat
    starts. Tokens outside every sequence hold `fill` (NaN by default, so a
    leak of padding into any result is visible)."""
    H, N = flat["r"].shape[1:]
    out = {}
    for name, arr in flat.items():
        dst = np.full((B * T, H, N), fill, dtype=np.float32)
        off = 0
        for st, L in zip(seq_start, lengths):
            dst[int(st):int(st) + int(L)] = arr[off:off + int(L)]
            off += int(L)
        out[name] = dst.reshape(B, T, H, N)
    inp = Inputs(dtype, out["r"], out["w"], out["k"], out["v"], out["a"], out["b"],
                 dy=out.get("dy"))
    inp.seq_start = np.asarray(seq_start, dtype=np.int32)
    inp.seq_len = np.asarray(lengths, dtype=np.int32)
    return inp


def checkpoint_bases(lengths) -> tuple[np.ndarray, int]:
    """First checkpoint slot of each sequence (exclusive prefix sum of
    ceil(len / CHUNK)) and the total number of slots."""
    n = (np.asarray(lengths, dtype=np.int64) + CHUNK - 1) // CHUNK
    base = np.concatenate([[0], np.cumsum(n)[:-1]]) if len(n) else np.zeros(0, np.int64)
    return base.astype(np.int32), int(n.sum())


def make_decode_inputs(B: int, H: int, N: int = 64, *, seed: int = 4, dtype: str = "bf16",
                       state_std: float = 0.1) -> Inputs:
    """One decode step: [B, 1, H, N] streams and a [B, H, N, N] state."""
    inp = make_inputs(B, 1, H, N, seed=seed, dtype=dtype)
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    inp.s0 = rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(state_std)
    return inp


@dataclasses.dataclass
class CEInputs:
    """Inputs of the linear-head cross-entropy: h [M, D] and W [V, D] hold
    bf16 values in fp32 arrays, targets [M] int32 (IGNORE on pad rows),
    dloss [M] fp32."""
    h: np.ndarray
    W: np.ndarray
    targets: np.ndarray
    dloss: np.ndarray


IGNORE = -100


def make_ce_inputs(M: int, D: int, V: int, *, seed: int = 5, logit_std: float = 2.0,
                   pad_frac: float = 0.05, dloss: str = "mean") -> CEInputs:
    """h ~ N(0, 1) (a normalised hidden state), W ~ N(0, (logit_std^2) / D)
    so the logits have standard deviation about logit_std, both rounded to
    bf16; targets uniform on [0, V) with a fraction pad_frac of rows set to
    IGNORE; dloss = 1 / (number of unmasked rows) on every row ("mean") or
    N(0, 1) ("normal")."""
    rng = np.random.Generator(np.random.PCG64(seed))
    h = round_bf16(rng.standard_normal((M, D), dtype=np.float32))
    W = round_bf16(rng.standard_normal((V, D), dtype=np.float32)
                   * np.float32(logit_std / np.sqrt(D)))
    t = rng.integers(0, V, size=M).astype(np.int32)
    t[rng.random(M) < pad_frac] = IGNORE
    if dloss == "mean":
        dl = np.full(M, 1.0 / max(1, int((t != IGNORE).sum())), dtype=np.float32)
    else:
        dl = rng.standard_normal(M, dtype=np.float32)
    return CEInputs(h, W, t, dl)


@dataclasses.dataclass
class GDNInputs:
    """One token of a gated DeltaNet layer: q, k [B, Hk, N] and v [B, H, N]
    (values of the I/O dtype held in fp32), g, beta [B, H] fp32, state
    [B, H, N, N] fp32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    s0: np.ndarray


def make_gdn_inputs(B: int, H: int, Hk: int, N: int = 128, *, seed: int = 8, dtype: str = "bf16",
                    state_std: float = 0.1) -> GDNInputs:
    """q, k, v ~ N(0, 1) rounded to dtype; g = -U(0.01, 1) (a log-decay);
    beta ~ U(0.05, 1) (a sigmoid output); state ~ N(0, state_std^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = round_to(rng.standard_normal((B, Hk, N), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((B, Hk, N), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((B, H, N), dtype=np.float32), dtype)
    g = (-rng.uniform(0.01, 1.0, (B, H))).astype(np.float32)
    beta = rng.uniform(0.05, 1.0, (B, H)).astype(np.float32)
    s0 = rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(state_std)
    return GDNInputs(q, k, v, g, beta, s0)


def make_gdn_sequence(B: int, T: int, H: int, Hk: int, N: int = 128, *, seed: int = 10,
                      dtype: str = "bf16", s0_std: float = 0.0) -> GDNInputs:
    """A dense batch of GDN tokens, q, k [B, T, Hk, N], v [B, T, H, N],
    g, beta [B, T, H], drawn as in make_gdn_inputs; s0 ~ N(0, s0_std^2)
    [B, H, N, N], or None when s0_std is 0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = round_to(rng.standard_normal((B, T, Hk, N), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((B, T, Hk, N), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((B, T, H, N), dtype=np.float32), dtype)
    g = (-rng.uniform(0.01, 1.0, (B, T, H))).astype(np.float32)
    beta = rng.uniform(0.05, 1.0, (B, T, H)).astype(np.float32)
    s0 = (rng.standard_normal((B, H, N, N), dtype=np.float32) * np.float32(s0_std)) if s0_std else None
    return GDNInputs(q, k, v, g, beta, s0)
