"""Benchmark of the WKV-7 hot path on one MI355X.

One step = the whole path over one synthetic batch of the training workload
(bf16 streams, fp32 state, B=4, T=4096, H=32, N=64, zero initial state,
dy ~ N(0,1)): wkv7_forward writing 16-token checkpoints, then wkv7_backward.
Inputs are resident in HBM before timing starts. The JSON line reports whole
step throughput in tokens/s (a token spans all H heads), the roofline of the
dominant kernel (HIP events on the launch stream), and the fp64 oracle timed
on the host's cores over a bounded sample of the same workload. Further
objects time the other calls of the library on their own workloads
(prefill, ragged batches, decode, the I/O variants, and the LM-head
cross-entropy over the 65536-entry vocabulary).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(path):
    import hashlib
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs, or None
    when there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or "sources" not in rec:
        return None
    for name, sha in rec["sources"].items():
        src = os.path.join(ROOT, "linear_recurrent_lm_amd", "csrc", name)
        if not os.path.exists(src) or source_digest(src) != sha:
            return None
    return rec["bytes_per_launch"]


def cpu_baseline(inp, budget_s):
    """fp64 oracle forward + backward on whole (b, h) units of the same
    workload until about budget_s seconds have been spent."""
    from oracle import oracle as O
    B, T, H, _ = inp.r.shape
    threads = O.max_threads()
    units = [(b, h) for b in range(B) for h in range(H)]
    done = 0
    t0 = time.perf_counter()
    while done < len(units) and time.perf_counter() - t0 < budget_s:
        batch = units[done:done + threads]
        for_b = {}
        for b, h in batch:
            for_b.setdefault(b, []).append(h)
        for b, hs in for_b.items():
            sl = [x[b:b + 1, :, hs] for x in inp.streams()]
            dy = inp.dy[b:b + 1, :, hs]
            O.forward(*sl, checkpoints=True, threads=threads)
            O.backward(*sl, dy=dy, threads=threads)
        done += len(batch)
    el = time.perf_counter() - t0
    tok_heads = done * T
    return {"value": tok_heads / H / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {B * H} (b,h) units x T={T}: fp64 forward with checkpoints + "
                      f"backward, {el:.1f} s"}


def _time_ms(fn, warmup, steps, ev):
    """Mean duration of fn() over `steps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    rec = []
    for _ in range(steps):
        e0, e1 = ev(), ev()
        e0.record()
        fn()
        e1.record()
        rec.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in rec]))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the kernels run on one GPU (units shard across GPUs without communication, which is not implemented here); --gpus must be 1"}))
        sys.exit(2)
    import torch
    from linear_recurrent_lm_amd import synth
    from linear_recurrent_lm_amd import wkv7 as W

    dev = "cuda:0"
    if args.copy_calibration:
        src = torch.empty(64 << 20, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4}), flush=True)
        return
    torch.cuda.set_device(0)
    W.lib()
    B, T, H = 4, 4096, 32
    inp = synth.make_inputs(B, T, H, N, seed=3, dtype="bf16", with_dy=True)
    ts = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in inp.streams()]
    dy = torch.from_numpy(inp.dy).to(dev).to(torch.bfloat16)
    y = torch.empty_like(ts[0])
    s_out = torch.empty((B, H, N, N), device=dev, dtype=torch.float32)
    ckpt = torch.empty((W.checkpoint_slots(B, T), H, N, N), device=dev, dtype=torch.float32)
    grads = {n: torch.empty_like(ts[0]) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    ws = torch.empty(W.wkv7_workspace_bytes(B, T, H, W.BF16), device=dev, dtype=torch.uint8)

    # Forward-only prefill workload (B=16, T=1024, H=32, random initial state).
    pin = synth.make_inputs(16, 1024, H, N, seed=2, dtype="bf16", s0_std=0.1)
    pts = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in pin.streams()]
    ps0 = torch.from_numpy(pin.s0).to(dev)
    py = torch.empty_like(pts[0])
    pso = torch.empty_like(ps0)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    fwd_ms, bwd_ms = [], []

    def step(record):
        e0, e1, e2 = ev(), ev(), ev()
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
    for e0, e1, e2 in recs:
        fwd_ms.append(e0.elapsed_time(e1))
        bwd_ms.append(e1.elapsed_time(e2))
    ms_step = wall * 1e3 / args.steps
    tok = B * T
    value = tok / (ms_step * 1e-3)

    # prefill forward timing
    for _ in range(args.warmup):
        W.wkv7_forward(*pts, ps0, y=py, s_out=pso)
    torch.cuda.synchronize()
    pre = []
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record()
        W.wkv7_forward(*pts, ps0, y=py, s_out=pso)
        e1.record()
        pre.append((e0, e1))
    torch.cuda.synchronize()
    pre_ms = float(np.mean([a.elapsed_time(b) for a, b in pre]))

    # Ragged forward: 64 sequences, lengths ~ U[16, 2048], packed in 4 streams
    # with a state reset at each sequence boundary.
    lengths = synth.ragged_lengths(64, 16, 2048, seed=4)
    flat, _ = synth.make_segment_inputs(lengths, H, N, seed=11, dtype="bf16")
    T_rg, st_rg, ln_rg = synth.packed_layout(lengths, 4)
    _, st_s, ln_s = synth.sorted_table(st_rg, ln_rg)
    rg = synth.scatter_segments(flat, lengths, st_rg, 4, T_rg, fill=0.0, dtype="bf16")
    rts = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in rg.streams()]
    seg = W.Segments(4, T_rg, st_s, ln_s, dev)
    ry = torch.empty_like(rts[0])
    rso = torch.empty((len(lengths), H, N, N), device=dev, dtype=torch.float32)
    ragged_ms = _time_ms(lambda: W.wkv7_forward(*rts, None, segments=seg, y=ry, s_out=rso),
                         args.warmup, args.steps, ev)
    rg_tok = int(np.sum(lengths))

    # Decode: one step at B=512, H=32 reading and writing a 64x64 fp32 state per (b, h).
    dinp = synth.make_decode_inputs(512, H, N, seed=4)
    dts = [torch.from_numpy(x[:, 0]).to(dev).to(torch.bfloat16) for x in dinp.streams()]
    ds_in = torch.from_numpy(dinp.s0).to(dev)
    ds_out = torch.empty_like(ds_in)
    dy_out = torch.empty_like(dts[0])
    dec_ms = _time_ms(lambda: W.wkv7_decode_step(*dts, ds_in, s_out=ds_out, y=dy_out),
                      args.warmup, args.steps, ev)
    dec_bytes = 512 * H * (2 * N * N * 4 + 7 * N * 2)

    # Fused decode: the same step carried through the per-head GroupNorm, the
    # bonus and the output gate (gate in, out instead of y).
    frng = np.random.Generator(np.random.PCG64(5004))
    fg = torch.from_numpy(synth.round_to(frng.uniform(0.0, 2.0, (512, H, N)).astype(np.float32),
                                         "bf16")).to(dev).to(torch.bfloat16)
    fln_w = torch.from_numpy((1.0 + 0.3 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    fln_b = torch.from_numpy((0.2 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    frk = torch.from_numpy((0.5 * frng.standard_normal((H, N))).astype(np.float32)).to(dev)
    fout = torch.empty_like(dts[0])
    fdec_ms = _time_ms(lambda: W.wkv7_decode_step_fused(*dts, ds_in, fg, fln_w, fln_b, frk, 64e-5,
                                                         s_out=ds_out, out=fout),
                       args.warmup, args.steps, ev)
    fdec_bytes = 512 * H * (2 * N * N * 4 + 8 * N * 2)

    # Launch cost of a decode loop: K fused steps at B=1, H=32 (state in place),
    # launched one by one, then replayed from one captured graph.
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

    loop_eager_ms = _time_ms(decode_loop, args.warmup, args.steps, ev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_loop()
    torch.cuda.current_stream().wait_stream(side)
    loop_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(loop_graph):
        decode_loop()
    loop_graph_ms = _time_ms(loop_graph.replay, args.warmup, args.steps, ev)

    # Gated DeltaNet decode through the RWKV-7 remap at GDN's layer geometry:
    # 32 value heads over 16 key heads, N = 128, B = 128 sequences, bf16.
    gin = synth.make_gdn_inputs(128, 32, 16, 128, seed=9, dtype="bf16")
    gq, gk, gv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (gin.q, gin.k, gin.v))
    gg, gb = torch.from_numpy(gin.g).to(dev), torch.from_numpy(gin.beta).to(dev)
    gs_in = torch.from_numpy(gin.s0).to(dev)
    gs_out = torch.empty_like(gs_in)
    gout = torch.empty_like(gv)
    del gin
    gdn_ms = _time_ms(lambda: W.wkv7_gdn_decode_step(gq, gk, gv, gg, gb, gs_in, s_out=gs_out, out=gout),
                      args.warmup, args.steps, ev)
    gdn_bytes = 128 * 32 * (2 * 128 * 128 * 4 + 2 * 128 * 2 + 8) + 128 * 16 * 2 * 128 * 2
    del gq, gk, gv, gg, gb, gs_in, gs_out, gout
    # GDN prefill through the remap: B=16, T=1024, same geometry. Per token and
    # value head: <S, k^> (2N^2), the update exp(g) S + c k^ (3N^2) and
    # <S, q^> (2N^2) flops.
    gsq = synth.make_gdn_sequence(16, 1024, 32, 16, 128, seed=11, dtype="bf16")
    sq, sk, sv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (gsq.q, gsq.k, gsq.v))
    sg, sb = torch.from_numpy(gsq.g).to(dev), torch.from_numpy(gsq.beta).to(dev)
    del gsq
    sout = torch.empty_like(sv)
    sws = torch.empty(W.wkv7_gdn_workspace_bytes(16, 1024, 16, 128), device=dev, dtype=torch.uint8)
    gdnf_ms = _time_ms(lambda: W.wkv7_gdn_forward(sq, sk, sv, sg, sb, None, out=sout, workspace=sws),
                       args.warmup, args.steps, ev)
    gdnf_flop = 7 * 128 * 128 * 16 * 1024 * 32
    del sq, sk, sv, sg, sb, sout, sws
    # The WKV-7 forward at head size 128 (token-order kernel), prefill shape.
    win = synth.make_inputs(16, 1024, 32, 128, seed=12, dtype="bf16", s0_std=0.1)
    wts = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in win.streams()]
    ws0 = torch.from_numpy(win.s0).to(dev)
    del win
    wy = torch.empty_like(wts[0])
    wso = torch.empty_like(ws0)
    f128_ms = _time_ms(lambda: W.wkv7_forward(*wts, ws0, y=wy, s_out=wso), args.warmup, args.steps, ev)
    f128_flop = 9 * 128 * 128 * 16 * 1024 * 32
    del wts, ws0, wy, wso

    # I/O variants: the prefill workload drawn in fp16; the training step with
    # w given as log(decay) and fp32 gradients.
    fin = synth.make_inputs(16, 1024, H, N, seed=2, dtype="f16", s0_std=0.1)
    fts = [torch.from_numpy(x).to(dev).to(torch.float16) for x in fin.streams()]
    fy = torch.empty_like(fts[0])
    f16_ms = _time_ms(lambda: W.wkv7_forward(*fts, ps0, y=fy, s_out=pso), args.warmup, args.steps, ev)
    del fts, fy
    lin = synth.make_inputs(B, T, H, N, seed=3, dtype="bf16", with_dy=True, decay="log")
    lts = [torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in lin.streams()]
    g32 = {n: torch.empty(lts[0].shape, device=dev, dtype=torch.float32) for n in grads}

    def log_step():
        W.wkv7_forward(*lts, None, checkpoints=True, y=y, s_out=s_out, ckpt=ckpt, decay="log")
        W.wkv7_backward(*lts, ckpt, dy, None, grads=g32, want_ds0=True, workspace=ws,
                        decay="log", grad_f32=True)

    log_ms = _time_ms(log_step, args.warmup, args.steps, ev)
    del lts, g32

    # Vocabulary cross-entropy of the LM head on the training batch's tokens:
    # M = 4 x 4096 rows, D = 2048 (the 1.5B width), V = 65536 (World
    # vocabulary), 5% pad rows, mean reduction; backward in vocabulary
    # chunks of 16384 rows. Flops as executed: 2MVD forward, 6MVD backward (the logits are
    # recomputed instead of stored).
    from linear_recurrent_lm_amd import vocab_ce as VC
    CM, CD, CV, CCH = B * T, 2048, 65536, 16384
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
    ce_f_ms = _time_ms(lambda: VC.vce_forward(ch, cw, ct, loss=closs, lse=clse, workspace=cfws),
                       args.warmup, args.steps, ev)
    ce_b_ms = _time_ms(lambda: VC.vce_backward(ch, cw, ct, clse, cdl, vocab_chunk=CCH, dh=cdh, dw=cdw,
                                               workspace=cbws), args.warmup, args.steps, ev)
    ce_flop = 2.0 * CM * CV * CD
    del ch, cw, ct, cdl, closs, clse, cdh, cdw, cfws, cbws

    f_ms, b_ms = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    th = tok * H
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

    def fracs(k):
        kk = kernels[k]
        t = kk["ms"] * 1e-3
        return {"ms": kk["ms"], "tokens_per_s": tok / t,
                "fp32_frac": kk["flop"] / t / PEAK_FP32, "hbm_frac": kk["bytes"] / t / PEAK_HBM}

    pre_th = 16 * 1024 * H
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "WKV-7 forward (16-token checkpoints) + backward, bf16 streams, "
                               "fp32 state, B=4 T=4096 H=32 N=64, zero initial state, dy~N(0,1)",
                   "global_batch": B, "seq_len": T, "heads": H, "head_size": N,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": {k: fracs(k) for k in kernels},
        "prefill_forward": {"workload": "bf16 B=16 T=1024 H=32, initial state N(0,0.1^2)",
                            "ms": pre_ms, "tokens_per_s": 16 * 1024 / (pre_ms * 1e-3),
                            "fp32_frac": FWD_FLOP * pre_th / (pre_ms * 1e-3) / PEAK_FP32,
                            "hbm_frac": FWD_BYTES * pre_th / (pre_ms * 1e-3) / PEAK_HBM},
    }
    out["ragged_forward"] = {"workload": "bf16 64 sequences, lengths ~ U[16, 2048] (%d tokens), packed in 4 "
                                         "streams with per-sequence resets, H=32" % rg_tok,
                             "ms": ragged_ms, "tokens_per_s": rg_tok / (ragged_ms * 1e-3),
                             "fp32_frac": FWD_FLOP * rg_tok * H / (ragged_ms * 1e-3) / PEAK_FP32}
    out["decode_step"] = {"workload": "bf16 B=512 T=1 H=32, fp32 state in and out",
                          "us": dec_ms * 1e3, "sequence_steps_per_s": 512 / (dec_ms * 1e-3),
                          "GB_per_s": dec_bytes / (dec_ms * 1e-3) / 1e9,
                          "hbm_frac": dec_bytes / (dec_ms * 1e-3) / PEAK_HBM}
    out["decode_step_fused"] = {
        "workload": "bf16 B=512 T=1 H=32, fp32 state in and out, then per-head GroupNorm, bonus and gate",
        "us": fdec_ms * 1e3, "sequence_steps_per_s": 512 / (fdec_ms * 1e-3),
        "GB_per_s": fdec_bytes / (fdec_ms * 1e-3) / 1e9,
        "hbm_frac": fdec_bytes / (fdec_ms * 1e-3) / PEAK_HBM}
    out["decode_loop_b1"] = {
        "workload": "bf16 B=1 H=32, %d fused steps with the state in place" % K,
        "us_per_step_launched": loop_eager_ms * 1e3 / K,
        "us_per_step_graph_replay": loop_graph_ms * 1e3 / K}
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
    out["prefill_forward_n128"] = {
        "workload": "WKV-7 forward at head size 128, bf16 B=16 T=1024 H=32, initial state N(0,0.1^2)",
        "ms": f128_ms, "tokens_per_s": 16 * 1024 / (f128_ms * 1e-3),
        "fp32_frac": f128_flop / (f128_ms * 1e-3) / PEAK_FP32}
    out["variants"] = {
        "prefill_forward_f16": {"workload": "fp16 B=16 T=1024 H=32, initial state N(0,0.1^2)",
                                "ms": f16_ms, "tokens_per_s": 16 * 1024 / (f16_ms * 1e-3),
                                "fp32_frac": FWD_FLOP * pre_th / (f16_ms * 1e-3) / PEAK_FP32},
        "train_step_log_decay_f32_grads": {
            "workload": "bf16 B=4 T=4096 H=32, w as log(decay), gradients in fp32 "
                        "(forward with checkpoints + backward)",
            "ms": log_ms, "tokens_per_s": tok / (log_ms * 1e-3)},
    }
    out["vocab_ce"] = {
        "workload": "LM-head cross-entropy, bf16 h [16384, 2048] and W [65536, 2048], 5% pad rows, "
                    "mean reduction, backward in vocabulary chunks of 16384 rows",
        "forward_ms": ce_f_ms, "backward_ms": ce_b_ms,
        "tokens_per_s": CM / ((ce_f_ms + ce_b_ms) * 1e-3),
        "forward_tflops": ce_flop / (ce_f_ms * 1e-3) / 1e12,
        "backward_tflops": 3 * ce_flop / (ce_b_ms * 1e-3) / 1e12,
        "mfma_bf16_frac": 4 * ce_flop / ((ce_f_ms + ce_b_ms) * 1e-3) / PEAK_BF16}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
