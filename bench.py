"""Benchmark of the WKV-7 hot path on one MI355X.

One step = the whole path over one synthetic batch of the training workload
(bf16 streams, fp32 state, B=4, T=4096, H=32, N=64, zero initial state,
dy ~ N(0,1)): wkv7_forward writing 16-token checkpoints, then wkv7_backward.
Inputs are resident in HBM before timing starts. The JSON line reports whole
step throughput in tokens/s (a token spans all H heads), the roofline of the
dominant call (HIP events on the launch stream), and the fp64 oracle timed
on the host's cores over a bounded sample of the same workload. Further
objects time the other calls of the library on their own workloads; each is
a "leg" that --only can select, so that a profiler run covers one leg:

    train     the step above (forward with checkpoints + backward)
    prefill   forward, B=16 T=1024 H=32, initial state N(0, 0.1^2)
    d768      forward, B=8 T=4096 H=12 (the D=768 model shape)
    small     forward, fp32 B=1 T=64 H=1 (launch-latency bound)
    ragged    64 sequences, lengths U[16, 2048]: packed in 4 streams and
              right-padded [64, 2048], forward; packed forward + backward
    decode    decode step B=512 H=32 (warm and after a 1 GiB cache flush),
              the fused step, and a B=1 loop launched and graph-replayed
    gdn       gated DeltaNet decode, prefill and its backward through the RWKV-7 remap
    n128      forward at head size 128; forward with checkpoints + backward
    variants  fp16 prefill; the step with log decay and fp32 gradients
    ce        LM-head cross-entropy over the 65536-entry vocabulary

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only LEG,...]
                    [--no-cpu-baseline] [--cpu-seconds S]
    python bench.py --summarize DIR     (no GPU: rocprofv3 output -> profiles/)
    python bench.py --copy-calibration  (a plain 256 MiB copy, for counter scaling)
    python bench.py --pipe-probe        (MFMA / VALU issue-pipe probe)
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WKV-7 tokens/sec fwd & fwd+bwd at H=32,N=64 bf16; % of HBM/FP32 roofline"
N = 64
# Algorithmic work of the token-order method per token-head.
FWD_FLOP = 9 * N * N            # 36,864
BWD_FLOP = 26 * N * N           # 106,496 (19 N^2 + 7 N^2 recompute)
FWD_BYTES = 6 * 128 + 128       # bf16 streams in, y out: 896
FWD_CKPT_BYTES = FWD_BYTES + 1024   # + one fp32 checkpoint per 16 tokens: 1920
BWD_BYTES = 6 * 128 + 128 + 1024 + 6 * 128  # 2688
PEAK_HBM = 8.0e12               # B/s
PEAK_FP32 = 157.3e12            # FLOP/s, vector or matrix fp32
PEAK_BF16 = 2.5e15              # FLOP/s, dense bf16 MFMA
LEGS = ("train", "prefill", "d768", "small", "ragged", "decode", "gdn", "n128", "variants", "ce")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--only", default="", help="comma-separated legs to run (default: all)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    p.add_argument("--pipe-probe", action="store_true",
                   help="only run the issue-pipe probe: MFMA waves and VALU waves sharing a SIMD")
    p.add_argument("--summarize", default="",
                   help="reduce rocprofv3 output under DIR into the tables of profiles/ (no GPU)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "linear_recurrent_lm_amd", "csrc")


def source_digest(path):
    import hashlib
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(call):
    """HBM bytes per call from the committed counter runs, or None when there
    is none or a kernel source of the call changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(call)
    except (OSError, ValueError):
        return None
    if not rec or "sources" not in rec:
        return None
    for name, sha in rec["sources"].items():
        src = os.path.join(CSRC, name)
        if not os.path.exists(src) or source_digest(src) != sha:
            return None
    return rec.get("bytes_per_call")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, budget_s):
    """The fp64 oracle (forward with checkpoints + backward) on whole (b, h)
    units of the training workload: median of 3 runs on all the cores the
    oracle's OpenMP uses and median of 3 on one core, each sample sized from
    a one-unit calibration so the six runs take about budget_s seconds."""
    from oracle import oracle as O
    B, T, H, _ = inp.r.shape
    streams = [np.ascontiguousarray(x, dtype=np.float64) for x in inp.streams()]
    dy = np.ascontiguousarray(inp.dy, dtype=np.float64)
    all_units = [(b, h) for b in range(B) for h in range(H)]
    threads = O.max_threads()

    def run(units, nthreads):
        t0 = time.perf_counter()
        O.forward(*streams, checkpoints=True, units=units, threads=nthreads)
        O.backward(*streams, dy=dy, units=units, threads=nthreads)
        return time.perf_counter() - t0

    t1 = run(all_units[:1], 1)
    per_run = budget_s / 6.0
    n_one = int(max(1, min(len(all_units), round(per_run / t1))))
    n_all = int(max(threads, min(len(all_units), round(per_run * threads / t1) // threads * threads)))
    n_all = min(n_all, len(all_units))
    all_t = sorted(run(all_units[:n_all], threads) for _ in range(3))
    one_t = sorted(run(all_units[:n_one], 1) for _ in range(3))
    v_all = n_all * T / H / all_t[1]
    v_one = n_one * T / H / one_t[1]
    return {"value": v_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_all} of {B * H} (b,h) units x T={T} of the training workload: fp64 forward "
                      f"with checkpoints + backward; median of 3 runs ({all_t[1]:.2f} s) on {threads} "
                      f"threads; one core: {n_one} units, median of 3 ({one_t[1]:.2f} s)",
            "value_one_core": v_one, "runs": 3, "cpu_model": cpu_model()}


def pipe_probe():
    """Whether VALU work progresses on a SIMD while another wave on it issues
    MFMAs (libwkv7_probe.so). Per MFMA kind: loop cycles of the MFMA waves
    alone, of the VALU waves alone (iterations sized to match), and of both
    running at once; both ~ max(alone) means the two overlap, both ~ sum
    means they share one issue pipe."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "linear_recurrent_lm_amd", "libwkv7_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run python -m linear_recurrent_lm_amd.build")
    L = ctypes.CDLL(path)
    L.wkv7_probe_pipe.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    L.wkv7_probe_pipe.restype = ctypes.c_int
    dev = "cuda:0"
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    rec = torch.zeros(blocks * 32, device=dev, dtype=torch.int64)
    sink = torch.zeros(blocks * 512, device=dev, dtype=torch.float32)

    def run(kind, mask, mi, vi):
        st = L.wkv7_probe_pipe(kind, mask, mi, vi, blocks, ctypes.c_void_p(rec.data_ptr()),
                               ctypes.c_void_p(sink.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"wkv7_probe_pipe failed: {st}")
        torch.cuda.synchronize()
        r = rec.view(blocks, 8, 4).cpu().numpy()
        cyc, rt, simd = r[:, :, 0], r[:, :, 1], (r[:, :, 2] >> 4) & 3
        paired = float(np.mean(simd[:, :4] == simd[:, 4:]))
        lo, hi = cyc[:, :4], cyc[:, 4:]
        # shader clock from the 100 MHz constant-rate counter
        mhz = float(np.median(cyc[cyc > 0] / np.maximum(rt[cyc > 0], 1))) * 100.0 if np.any(cyc > 0) else None
        return float(np.median(lo)), float(np.median(hi)), paired, mhz

    names = {0: "v_mfma_f32_16x16x4_f32", 1: "v_mfma_f32_32x32x2_f32", 2: "v_mfma_f32_16x16x32_bf16",
             4: "v_mfma_f32_16x16x16_bf16", 5: "v_mfma_f32_16x16x32_bf16 (eight chains)",
             6: "v_mfma_f32_16x16x32_bf16 (one chain)", 7: "v_mfma_f32_16x16x4_f32 (one chain)",
             3: "v_fma_f32 (second VALU wave)"}
    out = {"workgroups": blocks, "waves": "8 per workgroup: waves 0-3 MFMA (4 independent chains) or, for "
                                          "the last entry, fp32 FMA; waves 4-7 fp32 FMA (8 independent chains); "
                                          "wave w and w+4 share a SIMD"}
    for kind, name in names.items():
        mi = 8192 if kind == 3 else 2048
        run(kind, 1, mi, 0)
        m_alone, _, paired, mhz = run(kind, 1, mi, 0)
        _, v_probe, _, _ = run(kind, 2, 0, 4096)
        vi = max(1, int(round(4096 * m_alone / v_probe)))
        _, v_alone, _, _ = run(kind, 2, 0, vi)
        m_both, v_both, paired2, _ = run(kind, 3, mi, vi)
        per = 8 if kind == 3 else 4
        out[name] = {"first_side_instructions_per_wave": per * mi, "valu_fma_per_wave": 8 * vi,
                     "cycles_first_alone": m_alone, "cycles_valu_alone": v_alone,
                     "cycles_both_first_waves": m_both, "cycles_both_valu_waves": v_both,
                     "cycles_per_first_instruction": m_alone / (per * mi),
                     "cycles_per_valu_fma": v_alone / (8 * vi),
                     "both_over_max_alone": max(m_both, v_both) / max(m_alone, v_alone),
                     "simd_pairing": min(paired, paired2), "shader_clock_mhz": mhz}
    return out


# ----------------------------------------------------------------------------
# Timing helpers (HIP events on the current stream, which is the launch stream
# the binding passes to the library).

def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def _time_ms(fn, warmup, steps, between=None):
    """Mean duration of fn() over `steps` calls. `between`, if given, runs
    before each timed call, outside the events (a cache flush)."""
    import torch
    for _ in range(warmup):
        if between is not None:
            between()
        fn()
    torch.cuda.synchronize()
    rec = []
    for _ in range(steps):
        if between is not None:
            between()
        e0, e1 = _ev(), _ev()
        e0.record()
        fn()
        e1.record()
        rec.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in rec]))


def _dev_streams(inp, dtype):
    import torch
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    return [torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").to(tdt) for x in inp.streams()]


def _fwd_obj(workload, ms, tok, th, bytes_per_th=FWD_BYTES):
    t = ms * 1e-3
    return {"workload": workload, "ms": ms, "tokens_per_s": tok / t,
            "fp32_frac": FWD_FLOP * th / t / PEAK_FP32, "hbm_frac": bytes_per_th * th / t / PEAK_HBM,
            "roofline_frac": max(FWD_FLOP * th / PEAK_FP32, bytes_per_th * th / PEAK_HBM) / t}


# ----------------------------------------------------------------------------
# Legs

def leg_train(args, W, synth, out):
    import torch
    dev = "cuda:0"
    B, T, H = 4, 4096, 32
    inp = synth.make_inputs(B, T, H, N, seed=3, dtype="bf16", with_dy=True)
    ts = _dev_streams(inp, "bf16")
    dy = torch.from_numpy(inp.dy).to(dev).to(torch.bfloat16)
    y = torch.empty_like(ts[0])
    s_out = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
    ckpt = torch.empty((W.checkpoint_slots(B, T), H, N, N), device=dev, dtype=torch.float32)
    grads = {n: torch.empty_like(ts[0]) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    ws = torch.empty(W.wkv7_workspace_bytes(B, T, H, W.BF16), device=dev, dtype=torch.uint8)
    torch.cuda.synchronize()

    def step(record):
        e0, e1, e2 = _ev(), _ev(), _ev()
        e0.record()
        W.wkv7_forward(*ts, None, checkpoints=True, y=y, s_out=s_out, ckpt=ckpt)
        e1.record()
        W.wkv7_backward(*ts, ckpt, dy, None, grads=grads, want_ds0=True, workspace=ws)
        e2.record()
        if record is not None:
            record.append((e0, e1, e2))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in recs]))
    b_ms = float(np.mean([b.elapsed_time(c) for _, b, c in recs]))
    ms_step = wall * 1e3 / args.steps
    tok = B * T
    th = tok * H
    out.update({"value": tok / (ms_step * 1e-3), "ms_per_step": ms_step})
    kernels = {
        "wkv7_forward_ckpt": dict(ms=f_ms, flop=FWD_FLOP * th, bytes=FWD_CKPT_BYTES * th),
        "wkv7_backward": dict(ms=b_ms, flop=BWD_FLOP * th, bytes=BWD_BYTES * th),
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["ms"])
    dom = kernels[dom_name]
    t_hbm = dom["bytes"] / PEAK_HBM
    t_fp = dom["flop"] / PEAK_FP32
    if t_fp >= t_hbm:
        achieved = dom["flop"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32 / 1e12, "unit": "TFLOP/s"}
    else:
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom_name)
    roof["kernel"] = {"wkv7_backward": "wkv7_backward (dsweep_kernel + bwd_chunk_kernel)",
                      "wkv7_forward_ckpt": "wkv7_forward (fwd_ws_kernel)"}[dom_name]
    out["roofline"] = roof
    ks = {}
    for k, kk in kernels.items():
        t = kk["ms"] * 1e-3
        ks[k] = {"ms": kk["ms"], "tokens_per_s": tok / t, "fp32_frac": kk["flop"] / t / PEAK_FP32,
                 "hbm_frac": kk["bytes"] / t / PEAK_HBM,
                 "roofline_frac": max(kk["flop"] / PEAK_FP32, kk["bytes"] / PEAK_HBM) / t}
    out["kernels"] = ks
    return inp


def leg_prefill(args, W, synth, out):
    import torch
    B, T, H = 16, 1024, 32
    pin = synth.make_inputs(B, T, H, N, seed=2, dtype="bf16", s0_std=0.1)
    pts = _dev_streams(pin, "bf16")
    ps0 = torch.from_numpy(pin.s0).to("cuda:0")
    py = torch.empty_like(pts[0])
    pso = torch.empty_like(ps0)
    ms = _time_ms(lambda: W.wkv7_forward(*pts, ps0, y=py, s_out=pso), args.warmup, args.steps)
    out["prefill_forward"] = _fwd_obj("bf16 B=16 T=1024 H=32, initial state N(0,0.1^2)", ms, B * T, B * T * H)


def leg_d768(args, W, synth, out):
    import torch
    B, T, H = 8, 4096, 12
    inp = synth.make_inputs(B, T, H, N, seed=1, dtype="bf16")
    ts = _dev_streams(inp, "bf16")
    y = torch.empty_like(ts[0])
    so = torch.empty((B, H, N, N), device="cuda:0", dtype=torch.float32)
    ms = _time_ms(lambda: W.wkv7_forward(*ts, None, y=y, s_out=so), args.warmup, args.steps)
    out["d768_forward"] = _fwd_obj("bf16 B=8 T=4096 H=12 (D=768), zero initial state", ms, B * T, B * T * H)


def leg_small(args, W, synth, out):
    import torch
    inp = synth.make_inputs(1, 64, 1, N, seed=0, dtype="f32")
    ts = _dev_streams(inp, "f32")
    y = torch.empty_like(ts[0])
    so = torch.empty((1, 1, N, N), device="cuda:0", dtype=torch.float32)
    ms = _time_ms(lambda: W.wkv7_forward(*ts, None, y=y, s_out=so), args.warmup, max(args.steps, 50))
    out["small_forward"] = {"workload": "fp32 B=1 T=64 H=1, zero initial state (one unit: launch-latency "
                                        "bound)", "us": ms * 1e3}


def leg_ragged(args, W, synth, out):
    import torch
    dev = "cuda:0"
    H = 32
    lengths = synth.ragged_lengths(64, 16, 2048, seed=4)
    rg_tok = int(np.sum(lengths))
    flat, _ = synth.make_segment_inputs(lengths, H, N, seed=11, dtype="bf16", with_dy=True)
    # packed: 4 streams with a reset at every sequence boundary
    T_rg, st_rg, ln_rg = synth.packed_layout(lengths, 4)
    _, st_s, ln_s = synth.sorted_table(st_rg, ln_rg)
    rg = synth.scatter_segments(flat, lengths, st_rg, 4, T_rg, fill=0.0, dtype="bf16")
    rts = _dev_streams(rg, "bf16")
    rdy = torch.from_numpy(rg.dy).to(dev).to(torch.bfloat16)
    seg = W.Segments(4, T_rg, st_s, ln_s, dev)
    ry = torch.empty_like(rts[0])
    rso = torch.empty((len(lengths), H, N, N), device=dev, dtype=torch.float32)
    packed_ms = _time_ms(lambda: W.wkv7_forward(*rts, None, segments=seg, y=ry, s_out=rso),
                         args.warmup, args.steps)
    # the same sequences right-padded, one per row of [64, 2048]
    st_p, ln_p = synth.padded_layout(lengths, 2048)
    pd = synth.scatter_segments(flat, lengths, st_p, 64, 2048, fill=0.0, dtype="bf16")
    pts = _dev_streams(pd, "bf16")
    pseg = W.Segments(64, 2048, st_p, ln_p, dev)
    py = torch.empty_like(pts[0])
    padded_ms = _time_ms(lambda: W.wkv7_forward(*pts, None, segments=pseg, y=py, s_out=rso),
                         args.warmup, args.steps)
    del pts, py
    # packed forward with checkpoints + backward
    ck = torch.empty((seg.slots, H, N, N), device=dev, dtype=torch.float32)
    grads = {n: torch.empty_like(rts[0]) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    ws = torch.empty(W.wkv7_workspace_bytes(4, T_rg, H, W.BF16, seg), device=dev, dtype=torch.uint8)

    def train():
        W.wkv7_forward(*rts, None, segments=seg, checkpoints=True, y=ry, s_out=rso, ckpt=ck)
        W.wkv7_backward(*rts, ck, rdy, None, segments=seg, grads=grads, workspace=ws)

    train_ms = _time_ms(train, args.warmup, args.steps)
    th = rg_tok * H
    wl = "bf16 64 sequences, lengths ~ U[16, 2048] (%d tokens), H=32, zero initial states" % rg_tok
    out["ragged_forward"] = _fwd_obj(wl + ", packed in 4 streams with per-sequence resets", packed_ms,
                                     rg_tok, th)
    out["ragged_forward_padded"] = _fwd_obj(wl + ", right-padded [64, 2048] with lengths", padded_ms,
                                            rg_tok, th)
    out["ragged_train_step"] = {"workload": wl + ", packed; forward with checkpoints + backward",
                                "ms": train_ms, "tokens_per_s": rg_tok / (train_ms * 1e-3),
                                "fp32_frac": (FWD_FLOP + BWD_FLOP) * th / (train_ms * 1e-3) / PEAK_FP32}


def leg_decode(args, W, synth, out):
    import torch
    dev = "cuda:0"
    H = 32
    dinp = synth.make_decode_inputs(512, H, N, seed=4)
    dts = [torch.from_numpy(x[:, 0]).to(dev).to(torch.bfloat16) for x in dinp.streams()]
    ds_in = torch.from_numpy(dinp.s0).to(dev)
    ds_out = torch.empty_like(ds_in)
    dy_out = torch.empty_like(dts[0])
    dec = lambda: W.wkv7_decode_step(*dts, ds_in, s_out=ds_out, y=dy_out)
    dec_ms = _time_ms(dec, args.warmup, args.steps)
    # a 1 GiB write between steps evicts the 268 MB state from the caches
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    dec_cold_ms = _time_ms(dec, args.warmup, args.steps, between=lambda: flush.fill_(1.0))
    del flush
    dec_bytes = 512 * H * (2 * N * N * 4 + 7 * N * 2)

    frng = np.random.Generator(np.random.PCG64(5004))
    fg = torch.from_numpy(synth.round_to(frng.uniform(0.0, 2.0, (512, H, N)).astype(np.float32),
                                         "bf16")).to(dev).to(torch.bfloat16)
    fln_w = torch.from_numpy((1.0 + 0.3 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    fln_b = torch.from_numpy((0.2 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    frk = torch.from_numpy((0.5 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    fout = torch.empty_like(dts[0])
    fdec_ms = _time_ms(lambda: W.wkv7_decode_step_fused(*dts, ds_in, fg, fln_w, fln_b, frk, 64e-5,
                                                         s_out=ds_out, out=fout), args.warmup, args.steps)
    fdec_bytes = 512 * H * (2 * N * N * 4 + 8 * N * 2)

    # launch cost of a decode loop: K fused steps at B=1, H=32 (state in place),
    # launched one by one, then replayed from one captured graph
    K = 64
    sinp = synth.make_inputs(1, K, H, N, seed=6, dtype="bf16")
    lsteps = [[torch.from_numpy(np.ascontiguousarray(x[:, t])).to(dev).to(torch.bfloat16)
               for x in sinp.streams()] for t in range(K)]
    lstate = torch.zeros((1, H, N, N), device=dev, dtype=torch.float32)
    lg = torch.ones((1, H, N), device=dev, dtype=torch.bfloat16)
    louts = [torch.empty((1, H, N), device=dev, dtype=torch.bfloat16) for _ in range(K)]

    def decode_loop():
        for t in range(K):
            W.wkv7_decode_step_fused(*lsteps[t], lstate, lg, fln_w, fln_b, frk, 64e-5,
                                     s_out=lstate, out=louts[t])

    loop_eager_ms = _time_ms(decode_loop, args.warmup, args.steps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_loop()
    torch.cuda.current_stream().wait_stream(side)
    loop_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(loop_graph):
        decode_loop()
    loop_graph_ms = _time_ms(loop_graph.replay, args.warmup, args.steps)

    out["decode_step"] = {"workload": "bf16 B=512 T=1 H=32, fp32 state in and out",
                          "us": dec_ms * 1e3, "sequence_steps_per_s": 512 / (dec_ms * 1e-3),
                          "GB_per_s": dec_bytes / (dec_ms * 1e-3) / 1e9,
                          "hbm_frac": dec_bytes / (dec_ms * 1e-3) / PEAK_HBM,
                          "us_after_cache_flush": dec_cold_ms * 1e3,
                          "hbm_frac_after_cache_flush": dec_bytes / (dec_cold_ms * 1e-3) / PEAK_HBM}
    out["decode_step_fused"] = {
        "workload": "bf16 B=512 T=1 H=32, fp32 state in and out, then per-head GroupNorm, bonus and gate",
        "us": fdec_ms * 1e3, "sequence_steps_per_s": 512 / (fdec_ms * 1e-3),
        "GB_per_s": fdec_bytes / (fdec_ms * 1e-3) / 1e9,
        "hbm_frac": fdec_bytes / (fdec_ms * 1e-3) / PEAK_HBM}
    out["decode_loop_b1"] = {
        "workload": "bf16 B=1 H=32, %d fused steps with the state in place" % K,
        "us_per_step_launched": loop_eager_ms * 1e3 / K,
        "us_per_step_graph_replay": loop_graph_ms * 1e3 / K}


def leg_gdn(args, W, synth, out):
    import torch
    dev = "cuda:0"
    # decode at GDN's layer geometry: 32 value heads over 16 key heads, N = 128, B = 128
    gin = synth.make_gdn_inputs(128, 32, 16, 128, seed=9, dtype="bf16")
    gq, gk, gv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (gin.q, gin.k, gin.v))
    gg, gb = torch.from_numpy(gin.g).to(dev), torch.from_numpy(gin.beta).to(dev)
    gs_in = torch.from_numpy(gin.s0).to(dev)
    gs_out = torch.empty_like(gs_in)
    gout = torch.empty_like(gv)
    del gin
    gdn_ms = _time_ms(lambda: W.wkv7_gdn_decode_step(gq, gk, gv, gg, gb, gs_in, s_out=gs_out, out=gout),
                      args.warmup, args.steps)
    gdn_bytes = 128 * 32 * (2 * 128 * 128 * 4 + 2 * 128 * 2 + 8) + 128 * 16 * 2 * 128 * 2
    del gq, gk, gv, gg, gb, gs_in, gs_out, gout
    # prefill B=16, T=1024, same geometry. Per token and value head: <S, k^>
    # (2N^2), the update exp(g) S + c k^ (3N^2) and <S, q^> (2N^2) flops.
    gsq = synth.make_gdn_sequence(16, 1024, 32, 16, 128, seed=11, dtype="bf16")
    sq, sk, sv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (gsq.q, gsq.k, gsq.v))
    sg, sb = torch.from_numpy(gsq.g).to(dev), torch.from_numpy(gsq.beta).to(dev)
    del gsq
    sout = torch.empty_like(sv)
    sws = torch.empty(W.wkv7_gdn_workspace_bytes(16, 1024, 16, 128), device=dev, dtype=torch.uint8)
    gdnf_ms = _time_ms(lambda: W.wkv7_gdn_forward(sq, sk, sv, sg, sb, None, out=sout, workspace=sws),
                       args.warmup, args.steps)
    gdnf_flop = 7 * 128 * 128 * 16 * 1024 * 32
    # the backward on the same batch: gradients of out (dout ~ N(0, 1)) back to
    # q, k, v, g, beta through the remap and the normalisation
    sdo = torch.randn(sv.shape, device=dev, dtype=torch.float32, generator=torch.Generator(dev).manual_seed(12)).to(torch.bfloat16)
    bws = torch.empty(W.wkv7_gdn_backward_workspace_bytes(16, 1024, 32, 16, 128), device=dev, dtype=torch.uint8)
    gdnb_ms = _time_ms(lambda: W.wkv7_gdn_backward(sq, sk, sv, sg, sb, None, sdo, None, want_ds0=False,
                                                   workspace=bws), args.warmup, args.steps)
    del bws, sdo
    out["gdn_decode_step"] = {
        "workload": "gated DeltaNet via the RWKV-7 remap, bf16 B=128, 32 value heads over 16 key heads, "
                    "N=128, fp32 state in and out",
        "us": gdn_ms * 1e3, "sequence_steps_per_s": 128 / (gdn_ms * 1e-3),
        "GB_per_s": gdn_bytes / (gdn_ms * 1e-3) / 1e9,
        "hbm_frac": gdn_bytes / (gdn_ms * 1e-3) / PEAK_HBM}
    out["gdn_prefill_forward"] = {
        "workload": "gated DeltaNet via the RWKV-7 remap, bf16 B=16 T=1024, 32 value heads over 16 key "
                    "heads, N=128, zero initial state",
        "ms": gdnf_ms, "tokens_per_s": 16 * 1024 / (gdnf_ms * 1e-3),
        "fp32_frac": gdnf_flop / (gdnf_ms * 1e-3) / PEAK_FP32}
    out["gdn_prefill_backward"] = {
        "workload": "gated DeltaNet backward via the RWKV-7 remap, same batch, dout ~ N(0,1): remap to fp32 "
                    "streams, WKV-7 forward with checkpoints and backward at N=128, pull-back",
        "ms": gdnb_ms, "tokens_per_s": 16 * 1024 / (gdnb_ms * 1e-3),
        "fp32_frac_wkv7_backward_flops": 26 * 128 * 128 * 16 * 1024 * 32 / (gdnb_ms * 1e-3) / PEAK_FP32}


def leg_n128(args, W, synth, out):
    import torch
    win = synth.make_inputs(16, 1024, 32, 128, seed=12, dtype="bf16", s0_std=0.1)
    wts = _dev_streams(win, "bf16")
    ws0 = torch.from_numpy(win.s0).to("cuda:0")
    del win
    wy = torch.empty_like(wts[0])
    wso = torch.empty_like(ws0)
    f128_ms = _time_ms(lambda: W.wkv7_forward(*wts, ws0, y=wy, s_out=wso), args.warmup, args.steps)
    f128_flop = 9 * 128 * 128 * 16 * 1024 * 32
    out["prefill_forward_n128"] = {
        "workload": "WKV-7 forward at head size 128, bf16 B=16 T=1024 H=32, initial state N(0,0.1^2)",
        "ms": f128_ms, "tokens_per_s": 16 * 1024 / (f128_ms * 1e-3),
        "fp32_frac": f128_flop / (f128_ms * 1e-3) / PEAK_FP32}
    # training step at head size 128 on the same shape: forward with
    # checkpoints, then the backward from dy ~ N(0, 1) and the initial state
    B, T, H = 16, 1024, 32
    rng = np.random.default_rng(13)
    dy = torch.from_numpy(rng.standard_normal((B, T, H, 128), dtype=np.float32)).to("cuda:0").to(torch.bfloat16)
    ck = torch.empty((W.checkpoint_slots(B, T), H, 128, 128), device="cuda:0", dtype=torch.float32)
    grads = {n: torch.empty_like(wts[0]) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    ws = torch.empty(W.wkv7_workspace_bytes(B, T, H, W.BF16, n=128), device="cuda:0", dtype=torch.uint8)
    fc_ms = _time_ms(lambda: W.wkv7_forward(*wts, ws0, checkpoints=True, y=wy, s_out=wso, ckpt=ck),
                     args.warmup, args.steps)
    b_ms = _time_ms(lambda: W.wkv7_backward(*wts, ck, dy, None, grads=grads, want_ds0=True, workspace=ws),
                    args.warmup, args.steps)
    th = B * T * H
    out["train_n128"] = {
        "workload": "WKV-7 at head size 128, bf16 B=16 T=1024 H=32: forward with 16-token checkpoints, "
                    "then the backward (token order, one workgroup per sequence and head)",
        "forward_ckpt_ms": fc_ms, "backward_ms": b_ms, "tokens_per_s": B * T / ((fc_ms + b_ms) * 1e-3),
        "backward_fp32_frac": 26 * 128 * 128 * th / (b_ms * 1e-3) / PEAK_FP32}


def leg_variants(args, W, synth, out):
    import torch
    dev = "cuda:0"
    B, T, H = 16, 1024, 32
    fin = synth.make_inputs(B, T, H, N, seed=2, dtype="f16", s0_std=0.1)
    fts = _dev_streams(fin, "f16")
    fs0 = torch.from_numpy(fin.s0).to(dev)
    fy = torch.empty_like(fts[0])
    fso = torch.empty_like(fs0)
    f16_ms = _time_ms(lambda: W.wkv7_forward(*fts, fs0, y=fy, s_out=fso), args.warmup, args.steps)
    del fts, fy
    B, T = 4, 4096
    lin = synth.make_inputs(B, T, H, N, seed=3, dtype="bf16", with_dy=True, decay="log")
    lts = _dev_streams(lin, "bf16")
    ldy = torch.from_numpy(lin.dy).to(dev).to(torch.bfloat16)
    y = torch.empty_like(lts[0])
    s_out = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
    ckpt = torch.empty((W.checkpoint_slots(B, T), H, N, N), device=dev, dtype=torch.float32)
    g32 = {n: torch.empty(lts[0].shape, device=dev, dtype=torch.float32)
           for n in ("dr", "dw", "dk", "dv", "da", "db")}
    ws = torch.empty(W.wkv7_workspace_bytes(B, T, H, W.BF16), device=dev, dtype=torch.uint8)

    def log_step():
        W.wkv7_forward(*lts, None, checkpoints=True, y=y, s_out=s_out, ckpt=ckpt, decay="log")
        W.wkv7_backward(*lts, ckpt, ldy, None, grads=g32, want_ds0=True, workspace=ws,
                        decay="log", grad_f32=True)

    log_ms = _time_ms(log_step, args.warmup, args.steps)
    pre_th = 16 * 1024 * H
    out["variants"] = {
        "prefill_forward_f16": {"workload": "fp16 B=16 T=1024 H=32, initial state N(0,0.1^2)",
                                "ms": f16_ms, "tokens_per_s": 16 * 1024 / (f16_ms * 1e-3),
                                "fp32_frac": FWD_FLOP * pre_th / (f16_ms * 1e-3) / PEAK_FP32},
        "train_step_log_decay_f32_grads": {
            "workload": "bf16 B=4 T=4096 H=32, w as log(decay), gradients in fp32 "
                        "(forward with checkpoints + backward)",
            "ms": log_ms, "tokens_per_s": B * T / (log_ms * 1e-3)},
    }


def leg_ce(args, W, synth, out):
    """Cross-entropy of the LM head on the training batch's tokens: M = 4 x
    4096 rows, D = 2048 (the 1.5B width), V = 65536 (World vocabulary), 5% pad
    rows, mean reduction; backward in vocabulary chunks of 16384 rows.
    Algorithmic flops: 2MVD forward, 4MVD backward (dh and dW); the backward
    executes 6MVD, as it recomputes the logits instead of storing them."""
    import torch
    from linear_recurrent_lm_amd import vocab_ce as VC
    dev = "cuda:0"
    CM, CD, CV, CCH = 4 * 4096, 2048, 65536, 16384
    cin = synth.make_ce_inputs(CM, CD, CV, seed=7)
    ch = torch.from_numpy(cin.h).to(dev).to(torch.bfloat16)
    cw = torch.from_numpy(cin.W).to(dev).to(torch.bfloat16)
    ct = torch.from_numpy(cin.targets).to(dev)
    cdl = torch.from_numpy(cin.dloss).to(dev)
    del cin
    closs = torch.empty(CM, device=dev, dtype=torch.float32)
    clse = torch.empty_like(closs)
    cdh = torch.empty((CM, CD), device=dev, dtype=torch.float32)
    cdw = torch.empty((CV, CD), device=dev, dtype=torch.float32)
    cfws = torch.empty(VC.vce_forward_workspace_bytes(CM, CD, CV), device=dev, dtype=torch.uint8)
    cbws = torch.empty(VC.vce_backward_workspace_bytes(CM, CD, CV, CCH), device=dev, dtype=torch.uint8)
    f_ms = _time_ms(lambda: VC.vce_forward(ch, cw, ct, loss=closs, lse=clse, workspace=cfws),
                    args.warmup, args.steps)
    b_ms = _time_ms(lambda: VC.vce_backward(ch, cw, ct, clse, cdl, vocab_chunk=CCH, dh=cdh, dw=cdw,
                                            workspace=cbws), args.warmup, args.steps)
    mvd2 = 2.0 * CM * CV * CD
    out["vocab_ce"] = {
        "workload": "LM-head cross-entropy, bf16 h [16384, 2048] and W [65536, 2048], 5% pad rows, "
                    "mean reduction, backward in vocabulary chunks of 16384 rows",
        "forward_ms": f_ms, "backward_ms": b_ms,
        "tokens_per_s": CM / ((f_ms + b_ms) * 1e-3),
        "forward_tflops": mvd2 / (f_ms * 1e-3) / 1e12,
        "backward_tflops_algorithmic": 2 * mvd2 / (b_ms * 1e-3) / 1e12,
        "backward_tflops_executed": 3 * mvd2 / (b_ms * 1e-3) / 1e12,
        "mfma_bf16_frac": 3 * mvd2 / ((f_ms + b_ms) * 1e-3) / PEAK_BF16,
        "mfma_bf16_frac_basis": "algorithmic 6MVD (forward 2MVD + backward 4MVD) over forward + backward"}


# ----------------------------------------------------------------------------
# rocprofv3 output -> profiles/ (CPU only)

# (kernel name prefix, leg) -> what the dispatch is, for the tables
KERNEL_LABELS = {
    "fwd_ws_kernel": "WKV-7 forward, chunk form",
    "dsweep_kernel": "WKV-7 backward, pass 1: state-gradient sweep",
    "bwd_chunk_kernel": "WKV-7 backward, pass 2: per-chunk gradients",
    "zero_uncovered_kernel": "segment mode: zeros at uncovered tokens",
    "decode_kernel": "WKV-7 decode step",
    "decode128_kernel": "WKV-7 decode step, head size 128",
    "fwd_cf_kernel": "WKV-7 forward, head size 128 (chunk form, split-bf16 MFMA for bf16 streams)",
    "bwd128_kernel": "WKV-7 backward, head size 128 (token order, one workgroup per unit)",
    "gdn_decode_kernel": "gated DeltaNet decode step",
    "gdn_norm_kernel": "gated DeltaNet prefill: q^, k^ pre-pass",
    "gdn_fwd_kernel": "gated DeltaNet prefill: recurrence (token order; fp32 and fp16 I/O)",
    "gdn_cf_kernel": "gated DeltaNet prefill: recurrence in chunk form (bf16 I/O, split-bf16 MFMA)",
    "gdn_remap_kernel": "gated DeltaNet backward: remapped fp32 streams",
    "gdn_pull_value_kernel": "gated DeltaNet backward: dg, dbeta, dv",
    "gdn_pull_key_kernel": "gated DeltaNet backward: dq, dk through the normalisation",
    "gemm_kernel": "cross-entropy GEMM core",
    "combine_kernel": "cross-entropy: merge of the vocabulary splits",
    "transpose_pad_kernel": "cross-entropy: padded transpose",
}
LEG_WORKLOADS = {
    "train": "training B=4 T=4096 H=32 (forward with checkpoints + backward)",
    "prefill": "prefill B=16 T=1024 H=32, initial state N(0, 0.1^2)",
    "d768": "forward B=8 T=4096 H=12",
    "small": "forward fp32 B=1 T=64 H=1",
    "ragged": "64 sequences U[16, 2048], packed (4 streams) and right-padded [64, 2048]",
    "decode": "decode B=512 H=32; fused step; B=1 loop",
    "gdn": "gated DeltaNet decode B=128, prefill forward and backward B=16 T=1024 (32 value heads over 16 key heads, N=128)",
    "n128": "forward at head size 128, B=16 T=1024 H=32",
    "variants": "fp16 prefill; training step with log decay and fp32 gradients",
    "ce": "cross-entropy M=16384 D=2048 V=65536",
}


def _short(name):
    for pre in ("void ", "wkv7::", "(anonymous namespace)::", "vce::"):
        name = name.replace(pre, "")
    return name.split("(")[0].strip()


def _read_rows(pattern, ours=True):
    """Rows of the CSVs matching `pattern`; with ours, this library's kernels
    only (the runs also trace torch's own copy and fill kernels)."""
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as fh:
            for r in csv.DictReader(fh):
                if not ours or _short(r["Kernel_Name"]).split("<")[0] in KERNEL_LABELS:
                    rows.append(r)
    return rows


def _trace_table(d):
    """Per (kernel, grid): calls and duration statistics from a kernel trace."""
    rows = _read_rows(os.path.join(d, "**", "*kernel_trace.csv"))
    by = {}
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault(key, []).append(dur)
    return {k: {"calls": len(v), "avg_us": float(np.mean(v)), "min_us": float(np.min(v)),
                "max_us": float(np.max(v))} for k, v in by.items()}


def _counter_table(d, ours=True):
    """Per (kernel, grid): mean value per dispatch of every counter collected."""
    rows = _read_rows(os.path.join(d, "**", "*counter_collection.csv"), ours)
    per = {}
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
        disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
        per[key][r["Counter_Name"]][disp] = per[key][r["Counter_Name"]].get(disp, 0.0) + float(r["Counter_Value"])
    return {k: {c: float(np.mean(list(v.values()))) for c, v in cs.items()} for k, cs in per.items()}


def summarize(root):
    """Reduce the rocprofv3 runs under `root` into the tables of profiles/.

    Expected layout (each a separate rocprofv3 run; the profile files list
    the exact commands):
      root/kt/<leg>/            --kernel-trace --stats  over `bench.py --only <leg>`
      root/pmc_<set>/<leg>/     --pmc <counters>        over `bench.py --only <leg>`
      root/pmc_<set>/copy/      --pmc <counters>        over `bench.py --copy-calibration`
    Writes profiles/kernels__<leg>.md per leg and profiles/traffic.json."""
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    legs = sorted({os.path.basename(p.rstrip("/")) for p in glob.glob(os.path.join(root, "*", "*/"))} - {"copy"})
    pmc_sets = sorted(os.path.basename(p.rstrip("/")) for p in glob.glob(os.path.join(root, "pmc_*/")))
    # counter calibration: bytes a plain 256 MiB copy reads / writes per KiB counted
    scale = {}
    for s in pmc_sets:
        # the copy run's largest dispatch is the 256 MiB copy itself
        cal = _counter_table(os.path.join(root, s, "copy"), ours=False)
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = [cs[c] for cs in cal.values() if c in cs]
            if vals and max(vals) > 0:
                scale[c] = (256 << 20) / (max(vals) * 1024.0)
    traffic = {}
    written = []
    for leg in legs:
        trace = _trace_table(os.path.join(root, "kt", leg))
        counters = {}
        for s in pmc_sets:
            for key, cs in _counter_table(os.path.join(root, s, leg)).items():
                counters.setdefault(key, {}).update(cs)
        if not trace and not counters:
            continue
        keys = sorted(set(trace) | set(counters), key=lambda k: -trace.get(k, {}).get("avg_us", 0.0))
        lines = [f"# Kernels of the `{leg}` leg: {LEG_WORKLOADS.get(leg, leg)}", "",
                 "Commands (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):", "",
                 f"    rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof/kt/{leg} -o kt -- "
                 f"python3 bench.py --only {leg} --steps 5 --warmup 2 --no-cpu-baseline"]
        for s in pmc_sets:
            cset = sorted({c for cs in counters.values() for c in cs if c in PMC_SETS.get(s, ())})
            if cset:
                lines.append(f"    rocprofv3 --pmc {' '.join(PMC_SETS[s])} -f csv -d gpurun_out/prof/{s}/{leg} "
                             f"-o {s} -- python3 bench.py --only {leg} --steps 2 --warmup 1 --no-cpu-baseline")
        for s, c in (("pmc_fetch", "FETCH_SIZE"), ("pmc_write", "WRITE_SIZE")):
            if s in pmc_sets and c in scale:
                lines.append(f"    rocprofv3 --pmc {c} -f csv -d gpurun_out/prof/{s}/copy -o {s} -- "
                             f"python3 bench.py --copy-calibration")
        lines += ["", f"    python3 bench.py --summarize gpurun_out/prof", ""]
        lines += ["Durations are per dispatch from the kernel trace; counters are per dispatch (summed over the "
                  "chip's instances), from counter runs in which rocprofv3 serialises dispatches.", ""]
        lines += ["| kernel | grid (threads) | calls | avg (us) | min (us) | max (us) |",
                  "|---|---|---|---|---|---|"]
        for k in keys:
            t = trace.get(k)
            if t:
                lines.append(f"| `{k[0]}` | {k[1]} | {t['calls']} | {t['avg_us']:.1f} | {t['min_us']:.1f} | "
                             f"{t['max_us']:.1f} |")
        if counters:
            lines += ["", "Derived per dispatch. GRBM_GUI_ACTIVE arrives summed over the 8 XCDs, so the dispatch's "
                          "active cycles are GRBM_GUI_ACTIVE / 8 (this matches the traced durations at the "
                          "measured 2.1-2.2 GHz shader clock):",
                      "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs) (rocprof's MfmaUtil);",
                      "- VALU busy = SQ_ACTIVE_INST_VALU / (256 CUs x active cycles) (rocprof's VALUBusy);",
                      "- per wave = counter / SQ_WAVES;",
                      "- LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;",
                      "- wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;",
                      "- bytes = FETCH_SIZE, WRITE_SIZE (KiB) x the copy calibration factor "
                      + ", ".join(f"{c} {v:.3f}" for c, v in sorted(scale.items())) + ".", ""]
            cols = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM",
                    "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE", "FETCH_SIZE", "WRITE_SIZE"]
            lines += ["| kernel | grid | " + " | ".join(cols) + " |", "|---|---|" + "---|" * len(cols)]
            for k in keys:
                cs = counters.get(k)
                if not cs:
                    continue
                lines.append(f"| `{k[0]}` | {k[1]} | " + " | ".join(
                    (f"{cs[c]:.4g}" if c in cs else "-") for c in cols) + " |")
            lines += ["", "| kernel | grid | VALU / wave | MFMA / wave | LDS / wave | MFMA busy | VALU busy | "
                          "LDS conflict share | wait share | read (MB) | written (MB) |",
                      "|---|---|---|---|---|---|---|---|---|---|---|"]
            for k in keys:
                cs = counters.get(k)
                if not cs:
                    continue
                wv = cs.get("SQ_WAVES")
                g = cs.get("GRBM_GUI_ACTIVE")
                g = g / 8 if g else None

                def ratio(a, b, f=1.0):
                    return f"{f * cs[a] / b:.3g}" if (a in cs and b) else "-"
                rd = cs["FETCH_SIZE"] * 1024 * scale.get("FETCH_SIZE", 1.0) if "FETCH_SIZE" in cs else None
                wr = cs["WRITE_SIZE"] * 1024 * scale.get("WRITE_SIZE", 1.0) if "WRITE_SIZE" in cs else None
                lines.append(
                    f"| `{k[0]}` | {k[1]} | {ratio('SQ_INSTS_VALU', wv)} | {ratio('SQ_INSTS_MFMA', wv)} | "
                    f"{ratio('SQ_INSTS_LDS', wv)} | "
                    f"{ratio('SQ_VALU_MFMA_BUSY_CYCLES', g * 1024 if g else None)} | "
                    f"{ratio('SQ_ACTIVE_INST_VALU', g * 256 if g else None)} | "
                    f"{ratio('SQ_LDS_BANK_CONFLICT', cs.get('SQ_LDS_IDX_ACTIVE'))} | "
                    f"{ratio('SQ_WAIT_INST_ANY', cs.get('SQ_WAVE_CYCLES'))} | "
                    f"{'-' if rd is None else f'{rd / 1e6:.1f}'} | {'-' if wr is None else f'{wr / 1e6:.1f}'} |")
                if rd is not None and wr is not None:
                    traffic.setdefault(leg, {})[f"{k[0]}@{k[1]}"] = rd + wr
        path = os.path.join(prof, f"kernels__{leg}.md")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        written.append(path)
    # per-call traffic of the calls the roofline object reports
    calls = {}
    tr = traffic.get("train", {})
    fwd = [v for k, v in tr.items() if k.startswith("fwd_ws_kernel")]
    bwd = [v for k, v in tr.items() if k.startswith(("dsweep_kernel", "bwd_chunk_kernel"))]
    if fwd:
        calls["wkv7_forward_ckpt"] = {"bytes_per_call": fwd[0], "sources": _sources(["wkv7_forward.hip"])}
    if len(bwd) == 2:
        calls["wkv7_backward"] = {"bytes_per_call": sum(bwd),
                                  "sources": _sources(["wkv7_bwd_sweep.hip", "wkv7_backward.hip"])}
    if calls:
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(calls, fh, indent=1, sort_keys=True)
        written.append(TRAFFIC_FILE)
    return written


def _sources(names):
    shared = ["wkv7_mfma.h", "wkv7_device.h", "wkv7_kernels.h"]
    return {n: source_digest(os.path.join(CSRC, n)) for n in names + shared}


# Counter sets, one rocprofv3 run each (at most 8 SQ, 4 TCC and 2 GRBM
# counters per run).
PMC_SETS = {
    "pmc_inst": ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                 "SQ_INSTS_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"),
    "pmc_wait": ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES",
                 "SQ_WAIT_INST_LDS", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "GRBM_GUI_ACTIVE"),
    "pmc_fetch": ("FETCH_SIZE",),
    "pmc_write": ("WRITE_SIZE",),
}


# ----------------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize:
        for p in summarize(args.summarize):
            print(p)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the kernels run on one GPU (units shard across GPUs without communication, "
                                   "which is not implemented here); --gpus must be 1"}))
        sys.exit(2)
    import torch
    dev = "cuda:0"
    if args.pipe_probe:
        print(json.dumps({"pipe_probe": pipe_probe()}), flush=True)
        return
    if args.copy_calibration:
        src = torch.empty(64 << 20, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4}), flush=True)
        return
    from linear_recurrent_lm_amd import synth
    from linear_recurrent_lm_amd import wkv7 as W
    torch.cuda.set_device(0)
    W.lib()
    legs = [x for x in args.only.split(",") if x] if args.only else list(LEGS)
    bad = [x for x in legs if x not in LEGS]
    if bad:
        print(json.dumps({"error": f"unknown legs {bad}; legs are {list(LEGS)}"}))
        sys.exit(2)
    out = {
        "metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "WKV-7 forward (16-token checkpoints) + backward, bf16 streams, "
                               "fp32 state, B=4 T=4096 H=32 N=64, zero initial state, dy~N(0,1)",
                   "global_batch": 4, "seq_len": 4096, "heads": 32, "head_size": N,
                   "parallelism": "single GPU"},
        "roofline": None,
    }
    train_inp = None
    fns = {"train": leg_train, "prefill": leg_prefill, "d768": leg_d768, "small": leg_small,
           "ragged": leg_ragged, "decode": leg_decode, "gdn": leg_gdn, "n128": leg_n128,
           "variants": leg_variants, "ce": leg_ce}
    for leg in legs:
        print(f"bench: leg {leg}", file=sys.stderr, flush=True)
        r = fns[leg](args, W, synth, out)
        if leg == "train":
            train_inp = r
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline and train_inp is not None:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(train_inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
