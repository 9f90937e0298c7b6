#!/usr/bin/env python3
"""Benchmark of the DDTS hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunkwise-parallel forward (rodimus_ddts_chunk_fwd) over one
batch of the long-context prefill workload, the largest that runs on one GPU:
B=1 sequence x T=65536 tokens x H=16 heads, dk=64, dv=128, bf16 inputs, a
nonzero fp32 initial state, fp32 outputs.  The library splits each sequence
into segments (a transfer pass, an ordered combine, an output pass).  Inputs
are seeded synthetic tensors, resident in HBM before the timed region; the
step cycles through ``--rotate`` copies of them.

One JSON line on stdout:  value = tokens/s of the forward (B*T tokens per
step, whole call).  ``roofline`` is for the dominant kernel of the call (the
output pass): the call's algorithmic bytes (every input read once, the output
written once, the initial state read once; the output pass is the one launch
that reads all of them) over that pass's average duration, timed live with
HIP events that the library records on its own stream around each pass
(rodimus_trace_forward_events), next to the whole call's fraction.  The same
line carries the forward on the other workloads (the 130M and 1.6B layers,
each with its own fraction), the 130M layer fed low-rank beta_hat factors
(the fused path, and the bytes it saves), the decode-step bandwidth, the
backward (rodimus_ddts_chunk_bwd) on the 130M layer, a 24K-token prefill
followed by decode steps from its carried state, and the fp64 CPU oracle timed
on this host (all threads and one thread; a reported baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "DDTS chunk-fwd tokens/s + % MFMA/HBM roofline; decode-step state GB/s"
NAMES = ("q", "k", "v", "g", "tau", "beta_hat")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_long_prefill_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "gated_linear_attention_rodimus_amd", "csrc", "chunk_kernel.h")


def chunk_algorithmic(B, T, H, dk, dv, C, in_bytes=2, state_in=False, state_out=False):
    """Bytes the method must move and flops it must do (causal triangle once)."""
    ntok = B * T * H
    by = ntok * ((4 * dk + 2 * dv) * in_bytes + 4 * dv)
    by += (int(state_in) + int(state_out)) * B * H * dk * dv * 4
    fl = ntok * ((C + 1) * (dk + dv) + 4 * dk * dv)
    return by, fl


def swska_algorithmic(B, T, H, dk, dv, window, in_bytes=2):
    """Flops of the sliding-window shared-key attention (q . k and p v over
    each token's window, min(t + 1, window) keys) and the bytes it must move
    (q, v per token and head, the shared k per token, o fp32)."""
    keys = sum(min(t + 1, window) for t in range(T))
    fl = 2 * B * H * keys * (dk + dv)
    by = B * T * (H * (dk + dv) * in_bytes + dk * in_bytes + H * dv * 4)
    return by, fl


def decode_algorithmic(N, H, dk, dv, in_bytes=2):
    by = 2 * N * H * dk * dv * 4 + N * H * (4 * dk + 2 * dv) * in_bytes + N * H * dv * 4
    return by, 5 * N * H * dk * dv


def kernel_traffic(key):
    """HBM bytes per launch of one pass (``key``) from the committed rocprofv3
    counter summary, or None when the kernel source changed since the
    counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return rec["passes"][key]["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError, TypeError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_passes(R, call, n, stream):
    """Average duration (us) of each pass of ``n`` forward calls, from the
    events the library records around its launches."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    for row in evs:                      # create the events before handing them over
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(n):
        R.trace_forward_events(evs[i])
        call(i)
    R.trace_forward_events(None)
    torch.cuda.synchronize()
    return evs


def forward_sets(R, D, name, dev, rotate):
    """``rotate`` resident copies of a workload's inputs, outputs and state."""
    import torch
    wl = D.WORKLOADS[name]
    x = D.make(name)
    sets = []
    for r in range(max(1, rotate)):
        t = [x.torch(n, dev) for n in NAMES]
        if r:
            t = [a.clone() for a in t]
        out = torch.empty(wl.B, wl.T, wl.H, wl.dv, device=dev)
        fs = torch.empty(wl.B, wl.H, wl.dk, wl.dv, device=dev) if wl.final_state else None
        s0 = torch.from_numpy(x.initial_state).to(dev) if x.initial_state is not None else None
        sets.append((t, s0, out, fs))
    wsb = R.workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
    return x, sets, ws, wsb


def warm(step, seconds, min_steps=10):
    """Run ``step`` until it has kept the GPU busy for ``seconds`` (its clocks
    rise over the first ~20 ms under load)."""
    import torch
    i = 0
    tw = time.perf_counter()
    while i < min_steps or time.perf_counter() - tw < seconds:
        step(i)
        i += 1
        if i % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def timed(step, n, stream):
    """Average time (us) of ``n`` back-to-back calls, one event pair around
    them on ``stream`` (events between the calls would stall the queue)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=2, help="input copies cycled over steps")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--bwd-steps", type=int, default=20, help="timed backward calls (0: skip)")
    ap.add_argument("--serve-steps", type=int, default=100,
                    help="decode steps after a long prefill (0: skip)")
    ap.add_argument("--serve-prefill", type=int, default=24576)
    ap.add_argument("--serve-batch", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="long_prefill")
    ap.add_argument("--other-workloads", default="layer130m,layer1p6b",
                    help="comma-separated forward workloads timed after the main one "
                         "('none': skip)")
    ap.add_argument("--swska-steps", type=int, default=20,
                    help="timed calls of the sliding-window shared-key attention (0: skip)")
    ap.add_argument("--fused-steps", type=int, default=20,
                    help="timed calls of the 130M layer fed low-rank beta_hat factors (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times), "
                         "to scale the HBM byte counters of a profiler run")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": 2 * n * 4, "copies": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ddts_inputs as D
    import gated_linear_attention_rodimus_amd as R

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    wl = D.WORKLOADS[args.workload]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    x, sets, ws, wsb = forward_sets(R, D, args.workload, dev, args.rotate)
    plan = R.chunk_fwd_plan(B, T, H, dk, dv)
    torch.cuda.synchronize()

    def step(i):
        t, s0, out, fs = sets[i % len(sets)]
        R.chunk_fwd(*t, initial_state=s0, out=out, final_state=fs, workspace=ws)

    # warm-up: the W steps asked for, continued until the steps have kept the
    # GPU busy for 25 ms
    n_warm = 0
    for _ in range(args.warmup):
        step(n_warm)
        n_warm += 1
    torch.cuda.synchronize()
    n_warm += warm(step, 0.025)
    # the K timed steps: back to back on the library's stream (the current
    # one), a synchronize on each side for the wall clock and one event pair
    # for the device time
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    call_us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    value = B * T * args.steps / wall

    C = plan["chunk"]
    abytes, aflops = chunk_algorithmic(B, T, H, dk, dv, C, state_in=x.initial_state is not None,
                                       state_out=wl.final_state)
    # each pass of further calls, timed by the events the library records
    # around its own launches on its stream
    n_pass = max(5, args.steps)
    evs = time_passes(R, step, n_pass, stream)
    segmented = plan["segments"] > 1
    names = ("transfer", "combine", "output") if segmented else ("sweep",)
    passes = {}
    for j, nm in enumerate(names):
        passes[nm] = float(np.mean([row[j].elapsed_time(row[j + 1]) * 1e3 for row in evs]))
    dom = max(passes, key=passes.get)
    dom_us = passes[dom]
    ker = (f"chunk_fwd_kernel<{dk},{plan['dv_tile']},{C},bf16,outputs>"
           + (" (output pass of the segmented forward)" if segmented else " (one sweep)"))
    achieved = abytes / (dom_us * 1e-6) / 1e9
    traffic = kernel_traffic(dom)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": ker, "dominant_pass": dom,
                "algorithmic_bytes_per_launch": abytes,
                "launch_us": round(dom_us, 2),
                "passes_us": {k: round(v, 2) for k, v in passes.items()},
                "call_us": round(call_us, 2),
                "call_frac": round(abytes / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "traffic_over_algorithmic": (round(traffic / abytes, 4) if traffic else None),
                "mfma": {"achieved_tflops": round(aflops / (call_us * 1e-6) / 1e12, 2),
                         "peak_tflops": BF16_PEAK_TFLOPS,
                         "frac": round(aflops / (call_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops_per_call": aflops}}
    main_parity_sample = sets[0]
    del sets
    torch.cuda.empty_cache()

    # ---------------- the other forward workloads (the same timing: settled
    # clocks, one event pair around back-to-back calls, rotating input sets)
    others = {}
    names_o = [] if args.other_workloads in ("", "none") else args.other_workloads.split(",")
    for name in names_o:
        if name == args.workload:
            continue
        owl = D.WORKLOADS[name]
        ox, osets, ows, owsb = forward_sets(R, D, name, dev, 3)

        def ostep(i):
            t, s0_, out_, fs_ = osets[i % len(osets)]
            R.chunk_fwd(*t, initial_state=s0_, out=out_, final_state=fs_, workspace=ows)

        warm(ostep, 0.025)
        us = timed(ostep, 20, stream)
        oplan = R.chunk_fwd_plan(owl.B, owl.T, owl.H, owl.dk, owl.dv)
        oby, ofl = chunk_algorithmic(owl.B, owl.T, owl.H, owl.dk, owl.dv, oplan["chunk"],
                                     state_in=ox.initial_state is not None,
                                     state_out=owl.final_state)
        others[name] = {"shape": f"B={owl.B} T={owl.T} H={owl.H} dk={owl.dk} dv={owl.dv} bf16 inputs"
                                 + (", initial state" if ox.initial_state is not None else "")
                                 + (", returns S_T" if owl.final_state else ""),
                        "us_per_call": round(us, 2),
                        "tokens_per_s": round(owl.B * owl.T / (us * 1e-6), 1),
                        "algorithmic_bytes_per_call": oby,
                        "algorithmic_GBps": round(oby / us / 1e3, 1),
                        "frac_hbm": round(oby / us / 1e3 / HBM_PEAK_GBPS, 4),
                        "workspace_bytes": owsb, "plan": oplan}
        del osets, ows
        torch.cuda.empty_cache()

    # ---------------- the fused path: the 130M layer fed its rank-16 beta_hat
    # factors u, w (beta_hat = sigmoid(u w) formed in the chunk load)
    fused = None
    if args.fused_steps > 0:
        fwl = D.WORKLOADS["layer130m"]
        fx = D.make_fused("layer130m", conv_width=1)
        fsets = []
        for r in range(3):
            ft = {n: fx.torch(n, dev) for n in ("q", "k", "v", "g", "tau", "u", "w")}
            if r:
                ft = {n: a.clone() for n, a in ft.items()}
            fsets.append((ft, torch.empty(fwl.B, fwl.T, fwl.H, fwl.dv, device=dev)))

        def fstep(i):
            ft, fo = fsets[i % 3]
            R.chunk_fwd_fused(ft["q"], ft["k"], ft["v"], ft["g"], ft["tau"], u=ft["u"], w=ft["w"],
                              out=fo)

        warm(fstep, 0.025)
        fus = timed(fstep, args.fused_steps, stream)
        ntok = fwl.B * fwl.T * fwl.H
        r_ = fx.u.shape[-1]
        dense_by, _ = chunk_algorithmic(fwl.B, fwl.T, fwl.H, fwl.dk, fwl.dv, 64)
        fby = dense_by - ntok * 2 * fwl.dv * 2 + ntok * r_ * 2 + fwl.H * r_ * fwl.dv * 2
        fused = {"workload": f"layer130m B={fwl.B} T={fwl.T} H={fwl.H} dk={fwl.dk} dv={fwl.dv} bf16, "
                             f"beta_hat = sigmoid(u w) from rank-{r_} factors inside the kernel",
                 "us_per_call": round(fus, 2),
                 "tokens_per_s": round(fwl.B * fwl.T / (fus * 1e-6), 1),
                 "algorithmic_bytes_per_call": fby,
                 "bytes_saved_vs_dense_beta_hat": dense_by - fby,
                 "algorithmic_GBps": round(fby / fus / 1e3, 1),
                 "frac_hbm": round(fby / fus / 1e3 / HBM_PEAK_GBPS, 4)}
        del fsets
        torch.cuda.empty_cache()

    # ---------------- SW-SKA on a 1.6B-scale Rodimus+ layer
    swska = None
    if args.swska_steps > 0:
        sxw = D.make_swska("swska_1p6b")
        w_ = sxw.wl
        ssets = [[sxw.torch(n, dev) for n in ("q", "k", "v")] for _ in range(2)]
        so = torch.empty(w_.B, w_.T, w_.H, w_.dv, device=dev)
        sstep = lambda i: R.swska_fwd(*ssets[i % 2], w_.window, out=so)
        warm(sstep, 0.025)
        sus = timed(sstep, args.swska_steps, stream)
        sby, sfl = swska_algorithmic(w_.B, w_.T, w_.H, w_.dk, w_.dv, w_.window)
        swska = {"workload": f"swska_1p6b: B={w_.B} T={w_.T} H={w_.H} dk={w_.dk} dv={w_.dv} bf16, "
                             f"one shared key, window {w_.window}, fp32 out",
                 "us_per_call": round(sus, 2),
                 "tokens_per_s": round(w_.B * w_.T / (sus * 1e-6), 1),
                 "algorithmic_flops_per_call": sfl,
                 "tflops": round(sfl / (sus * 1e-6) / 1e12, 1),
                 "frac_mfma_bf16": round(sfl / (sus * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "algorithmic_bytes_per_call": sby,
                 "frac_hbm": round(sby / sus / 1e3 / HBM_PEAK_GBPS, 4)}
        del ssets, so
        torch.cuda.empty_cache()

    # ---------------- decode: back-to-back steps over resident states
    decode = None
    if args.decode_steps > 0:
        dsets, st = D.make_decode_pool("decode_batch")
        N, Hd, dkd, dvd = st.shape
        dins = [[s.torch(n, dev)[:, 0] for n in NAMES] for s in dsets]
        S = torch.from_numpy(st).to(dev)
        o = torch.empty(N, Hd, dvd, device=dev)
        for i in range(10):
            R.decode_step(*dins[i % len(dins)], S, out=o)
        torch.cuda.synchronize()
        us = timed(lambda i: R.decode_step(*dins[i % len(dins)], S, out=o), args.decode_steps, stream)
        dbytes, dflops = decode_algorithmic(N, Hd, dkd, dvd)
        # cold variant: state batches in rotation whose total (12 x 134 MB) exceeds
        # the 256 MB last-level cache, as when every layer of a model keeps a state
        n_cold = 12
        Ss = [S] + [S.clone() for _ in range(n_cold - 1)]
        us_cold = timed(lambda i: R.decode_step(*dins[i % len(dins)], Ss[i % n_cold], out=o),
                        args.decode_steps, stream)
        decode = {"workload": f"decode_batch N{N} H{Hd} dk{dkd} dv{dvd} bf16 inputs, fp32 state",
                  "steps": args.decode_steps, "us_per_step": round(us, 2),
                  "algorithmic_bytes_per_step": dbytes,
                  "state_GBps": round(2 * N * Hd * dkd * dvd * 4 / us / 1e3, 1),
                  "algorithmic_GBps": round(dbytes / us / 1e3, 1),
                  "frac_hbm": round(dbytes / us / 1e3 / HBM_PEAK_GBPS, 4),
                  "cold_us_per_step": round(us_cold, 2),
                  "cold_state_sets": n_cold,
                  "cold_algorithmic_GBps": round(dbytes / us_cold / 1e3, 1),
                  "cold_frac_hbm": round(dbytes / us_cold / 1e3 / HBM_PEAK_GBPS, 4),
                  "tokens_per_s": round(N / (us * 1e-6), 1)}
        del Ss, S
        torch.cuda.empty_cache()

    # ---------------- backward of the chunk forward on the 130M layer
    backward = None
    if args.bwd_steps > 0:
        bwl = D.WORKLOADS["layer130m"]
        Bb, Tb, Hb, dkb, dvb = bwl.B, bwl.T, bwl.H, bwl.dk, bwl.dv
        bx = D.make("layer130m")
        bt = [bx.torch(n, dev) for n in NAMES]
        rng = np.random.default_rng(2)
        d_out = torch.from_numpy(rng.standard_normal((Bb, Tb, Hb, dvb), dtype=np.float32)).to(dev)
        bwsb = R.bwd_workspace_bytes(Bb, Tb, Hb, dkb, dvb)
        bws = torch.empty(max(bwsb, 1), dtype=torch.uint8, device=dev)
        bstep = lambda i: R.chunk_bwd(*bt, d_out, workspace=bws)
        warm(bstep, 0.05, min_steps=2)
        bus = timed(bstep, args.bwd_steps, stream)
        ntok = Bb * Tb * Hb
        bbytes = ntok * ((4 * dkb + 2 * dvb) * 2 + 4 * dvb + (4 * dkb + 2 * dvb) * 4)
        backward = {"entry": "rodimus_ddts_chunk_bwd (state sweeps + chunk gradients)",
                    "workload": "layer130m", "calls": args.bwd_steps,
                    "us_per_call": round(bus, 1), "tokens_per_s": round(Bb * Tb / (bus * 1e-6), 1),
                    "algorithmic_bytes_per_call": bbytes,
                    "algorithmic_GBps": round(bbytes / bus / 1e3, 1),
                    "frac_hbm": round(bbytes / bus / 1e3 / HBM_PEAK_GBPS, 4),
                    "workspace_bytes": bwsb}
        del bt, bws, d_out
        torch.cuda.empty_cache()

    # ---------------- prefill then batched decode from the carried state
    serving = None
    if args.serve_steps > 0:
        sx = D.make("decode_batch", B=args.serve_batch, T=args.serve_prefill + 1, H=16)
        st_ = [sx.torch(n, dev) for n in NAMES]
        pre = [a[:, :args.serve_prefill].contiguous() for a in st_]
        tok = [a[:, args.serve_prefill].contiguous() for a in st_]
        s0 = torch.from_numpy(sx.initial_state).to(dev)
        Bs, Hs = sx.wl.B, sx.wl.H
        o_pre = torch.empty(Bs, args.serve_prefill, Hs, sx.wl.dv, device=dev)
        Sst = torch.empty(Bs, Hs, sx.wl.dk, sx.wl.dv, device=dev)
        o_dec = torch.empty(Bs, Hs, sx.wl.dv, device=dev)
        swsb = R.workspace_bytes(Bs, args.serve_prefill, Hs, sx.wl.dk, sx.wl.dv)
        sws = torch.empty(max(swsb, 1), dtype=torch.uint8, device=dev) if swsb else None
        R.chunk_fwd(*pre, initial_state=s0, out=o_pre, final_state=Sst, workspace=sws)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        R.chunk_fwd(*pre, initial_state=s0, out=o_pre, final_state=Sst, workspace=sws)
        e1.record(stream)
        for _ in range(args.serve_steps):
            R.decode_step(*tok, Sst, out=o_dec)
        e2.record(stream)
        torch.cuda.synchronize()
        pre_ms = e0.elapsed_time(e1)
        dec_us = e1.elapsed_time(e2) * 1e3 / args.serve_steps
        # the same decode steps captured once in a HIP graph and replayed (a
        # step this small is bound by launch overhead, which the graph removes;
        # the replay keeps advancing the carried state in place)
        def dec_loop():
            for _ in range(args.serve_steps):
                R.decode_step(*tok, Sst, out=o_dec)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            dec_loop()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dec_loop()
        graph.replay()
        torch.cuda.synchronize()
        e1.record(stream)
        graph.replay()
        e2.record(stream)
        torch.cuda.synchronize()
        dec_graph_us = e1.elapsed_time(e2) * 1e3 / args.serve_steps
        serving = {"workload": f"prefill {args.serve_prefill} tokens x {Bs} sequences x {Hs} heads "
                               f"(dk {sx.wl.dk}, dv {sx.wl.dv}, bf16), then {args.serve_steps} decode "
                               "steps from the carried state",
                   "prefill_ms": round(pre_ms, 3),
                   "prefill_tokens_per_s": round(Bs * args.serve_prefill / (pre_ms * 1e-3), 1),
                   "decode_us_per_step": round(dec_us, 2),
                   "decode_tokens_per_s": round(Bs / (dec_us * 1e-6), 1),
                   "decode_graph_us_per_step": round(dec_graph_us, 2),
                   "decode_graph_tokens_per_s": round(Bs / (dec_graph_us * 1e-6), 1)}

    # ---------------- CPU baseline: the fp64 oracle on this host, a bounded
    # sample of the same workload (whole sequences of some heads), once on all
    # threads and once on one thread; tokens/s counts B*T tokens of all H heads
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        hs = min(H, max(1, nthreads))          # heads in the sample: one per thread
        Ts = min(T, 16384)
        ins = [np.ascontiguousarray(x.f32(n)[:1, :Ts, :hs]) for n in NAMES]
        s0 = None if x.initial_state is None else np.ascontiguousarray(x.initial_state[:1, :hs])

        def rate(threads, heads, budget):
            sl = [np.ascontiguousarray(a[:, :, :heads]) for a in ins]
            s0s = None if s0 is None else np.ascontiguousarray(s0[:, :heads])
            passes, c0, ro = 0, time.perf_counter(), None
            while passes == 0 or time.perf_counter() - c0 < budget:
                o_, _ = oracle.fwd(*sl, s0s, nthreads=threads)
                ro = o_ if ro is None else ro
                passes += 1
            cs = time.perf_counter() - c0
            # token-heads per second, expressed as tokens of all H heads
            return passes * Ts * heads / cs / H, oracle.fwd.last_threads, passes, cs, ro

        v_all, used, p_all, c_all, ro = rate(nthreads, hs, 10.0)
        v_one, _, p_one, c_one, _ = rate(1, 1, 5.0)
        cpu = {"value": round(v_all, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
               "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
               "one_thread": {"value": round(v_one, 1), "unit": "tokens/s", "cores": 1,
                              "sample": f"1 head x {Ts} tokens, {p_one} passes, {c_one:.1f} s"},
               "sample": f"{args.workload}: first {Ts} tokens of {hs} of {H} heads (B=1), "
                         f"{p_all} passes, fp64 C oracle, {c_all:.1f} s; tokens/s counts "
                         f"token-heads / {H}"}
        gpu_o = main_parity_sample[2][:1, :Ts, :hs].cpu().numpy()
        # the GPU's first Ts tokens depend only on the first Ts tokens and S_0
        parity = {"max_abs_over_rms": oracle.rel_to_rms_error(gpu_o, ro), "bar": 1e-2,
                  "sample": "the CPU-baseline sample"}

    line = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "warmup_run": n_warm,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{args.workload}: B={B} T={T} H={H} dk={dk} dv={dv} "
                                   f"bf16 inputs, fp32 out/state"
                                   + (", initial state" if x.initial_state is not None else "")
                                   + (", returns S_T" if wl.final_state else "")
                                   + f"; plan: chunk {C}, dv tile {plan['dv_tile']}, "
                                     f"{plan['segments']} segments",
                       "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                       "rotating_input_sets": args.rotate, "parallelism": "single GPU"},
            "roofline": roofline, "cpu_baseline": cpu, "other_forward": others or None,
            "fused": fused, "swska": swska, "decode": decode, "backward": backward, "serving": serving,
            "parity": parity}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
