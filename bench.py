#!/usr/bin/env python3
"""Benchmark of the DDTS hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunkwise-parallel forward (rodimus_ddts_chunk_fwd) over one
batch of the 130M-scale layer workload: B=8 sequences x T=2048 tokens x H=12
heads, dk=64, dv=128, bf16 inputs, fp32 outputs.  Inputs are seeded synthetic
tensors, resident in HBM before the timed region; the step cycles through
``--rotate`` copies of them so that the 256 MB last-level cache cannot serve a
batch from the previous step.  After the chunk steps the same run times
``--decode-steps`` back-to-back decode steps over 256 x 16 resident fp32
states (the batched decode workload) and reports the state bandwidth, once on
one resident state batch (which the 256 MB last-level cache partly holds) and
once cold, rotating over 12 state batches (1.6 GB).

One JSON line on stdout:  value = tokens/s of the chunk forward (B*T tokens
per step), the roofline of the chunk kernel (HBM-bound: algorithmic bytes per
launch / its HIP-event-timed duration), the forward on the other workloads
(``--other-workloads``: the 1.6B-scale layer and the 64K-token prefill, both
segmented; time per call and algorithmic bandwidth), the decode-step bandwidth, the
backward (rodimus_ddts_chunk_bwd) on the same batch, a 24K-token prefill
followed by decode steps from its carried state, and the fp64 CPU oracle
timed on this host on the same workload (a reported baseline).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_layer130m_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "gated_linear_attention_rodimus_amd", "csrc", "chunk_kernel.h")


def chunk_algorithmic(B, T, H, dk, dv, C, in_bytes=2, state_in=False, state_out=False):
    """Bytes the method must move and flops it must do (causal triangle once)."""
    ntok = B * T * H
    by = ntok * ((4 * dk + 2 * dv) * in_bytes + 4 * dv)
    by += (int(state_in) + int(state_out)) * B * H * dk * dv * 4
    fl = ntok * ((C + 1) * (dk + dv) + 4 * dk * dv)
    return by, fl


def decode_algorithmic(N, H, dk, dv, in_bytes=2):
    by = 2 * N * H * dk * dv * 4 + N * H * (4 * dk + 2 * dv) * in_bytes + N * H * dv * 4
    return by, 5 * N * H * dk * dv


def kernel_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return rec["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=3, help="input copies cycled over steps")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--bwd-steps", type=int, default=20, help="timed backward calls (0: skip)")
    ap.add_argument("--serve-steps", type=int, default=100,
                    help="decode steps after a long prefill (0: skip)")
    ap.add_argument("--serve-prefill", type=int, default=24576)
    ap.add_argument("--serve-batch", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="layer130m")
    ap.add_argument("--other-workloads", default="layer1p6b,long_prefill",
                    help="comma-separated forward workloads timed after the main one "
                         "('none': skip)")
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
    wl = D.WORKLOADS[args.workload]
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    x = D.make(args.workload)
    sets = []
    for r in range(max(1, args.rotate)):
        t = [x.torch(n, dev) for n in NAMES]
        if r:
            t = [a.clone() for a in t]
        out = torch.empty(B, T, H, dv, device=dev)
        fs = torch.empty(B, H, dk, dv, device=dev) if wl.final_state else None
        s0 = torch.from_numpy(x.initial_state).to(dev) if x.initial_state is not None else None
        sets.append((t, s0, out, fs))
    wsb = R.workspace_bytes(B, T, H, dk, dv)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
    torch.cuda.synchronize()

    def step(i):
        t, s0, out, fs = sets[i % len(sets)]
        R.chunk_fwd(*t, initial_state=s0, out=out, final_state=fs, workspace=ws)

    # warm-up: the W steps asked for, continued until the steps have kept the
    # GPU busy for 25 ms (its clocks rise over the first ~20 ms under load:
    # 119 us per step measured after 5 warm-up steps, 105-106 us after 200 or
    # more)
    n_warm = 0
    tw = time.perf_counter()
    for _ in range(args.warmup):
        step(n_warm)
        n_warm += 1
    torch.cuda.synchronize()
    while time.perf_counter() - tw < 0.025:
        for _ in range(10):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    # the K launches go back to back on the library's stream (the current
    # one); one event pair brackets them, so the average launch duration is
    # (end - start) / K, gaps between launches included.  Events recorded
    # between the launches themselves stall the queue (~14 us per step here)
    # and would be timed as part of the kernel.
    stream = torch.cuda.current_stream(dev)
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
    avg_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    tokens = B * T
    value = tokens * args.steps / wall

    C = 64
    abytes, aflops = chunk_algorithmic(B, T, H, dk, dv, C, state_in=x.initial_state is not None,
                                       state_out=wl.final_state)
    achieved = abytes / avg_launch_s / 1e9
    traffic = kernel_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "chunk_fwd_kernel<64,64,64,bf16,outputs>" if wsb == 0 else "chunk_fwd (segmented)",
                "algorithmic_bytes_per_launch": abytes,
                "launch_us": round(avg_launch_s * 1e6, 2),
                "mfma": {"achieved_tflops": round(aflops / avg_launch_s / 1e12, 2),
                         "peak_tflops": BF16_PEAK_TFLOPS,
                         "frac": round(aflops / avg_launch_s / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops_per_launch": aflops}}

    # ---------------- the other forward workloads (the same timing: settled
    # clocks, one event pair around back-to-back calls, two rotating input sets)
    others = {}
    names = [] if args.other_workloads in ("", "none") else args.other_workloads.split(",")
    for name in names:
        if name == args.workload:
            continue
        owl = D.WORKLOADS[name]
        ox = D.make(name)
        osets = []
        for r in range(2):
            t = [ox.torch(n, dev) for n in NAMES]
            if r:
                t = [a.clone() for a in t]
            o_out = torch.empty(owl.B, owl.T, owl.H, owl.dv, device=dev)
            o_fs = torch.empty(owl.B, owl.H, owl.dk, owl.dv, device=dev) if owl.final_state else None
            o_s0 = torch.from_numpy(ox.initial_state).to(dev) if ox.initial_state is not None else None
            osets.append((t, o_s0, o_out, o_fs))
        owsb = R.workspace_bytes(owl.B, owl.T, owl.H, owl.dk, owl.dv)
        ows = torch.empty(max(owsb, 1), dtype=torch.uint8, device=dev) if owsb else None

        def ostep(i):
            t, s0_, out_, fs_ = osets[i % 2]
            R.chunk_fwd(*t, initial_state=s0_, out=out_, final_state=fs_, workspace=ows)

        i = 0
        tw = time.perf_counter()
        while i < 10 or time.perf_counter() - tw < 0.025:
            ostep(i)
            i += 1
            torch.cuda.synchronize()
        k = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(k):
            ostep(j)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / k
        oby, _ = chunk_algorithmic(owl.B, owl.T, owl.H, owl.dk, owl.dv, 64,
                                   state_in=ox.initial_state is not None, state_out=owl.final_state)
        others[name] = {"shape": f"B={owl.B} T={owl.T} H={owl.H} dk={owl.dk} dv={owl.dv} bf16 inputs"
                                 + (", initial state" if ox.initial_state is not None else "")
                                 + (", returns S_T" if owl.final_state else ""),
                        "us_per_call": round(us, 2),
                        "tokens_per_s": round(owl.B * owl.T / (us * 1e-6), 1),
                        "algorithmic_bytes_per_call": oby,
                        "algorithmic_GBps": round(oby / us / 1e3, 1),
                        "frac_hbm": round(oby / us / 1e3 / HBM_PEAK_GBPS, 4),
                        "workspace_bytes": owsb,
                        "plan": R.chunk_fwd_plan(owl.B, owl.T, owl.H, owl.dk, owl.dv)}
        del osets, ows
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.decode_steps):
            R.decode_step(*dins[i % len(dins)], S, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        dbytes, dflops = decode_algorithmic(N, Hd, dkd, dvd)
        # cold variant: state batches in rotation whose total (12 x 134 MB) exceeds
        # the 256 MB last-level cache, as when every layer of a model keeps a state
        n_cold = 12
        Ss = [S] + [S.clone() for _ in range(n_cold - 1)]
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.decode_steps):
            R.decode_step(*dins[i % len(dins)], Ss[i % n_cold], out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        us_cold = e0.elapsed_time(e1) * 1e3 / args.decode_steps
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

    # ---------------- backward of the chunk forward on the same batch
    backward = None
    if args.bwd_steps > 0:
        rng = np.random.default_rng(2)
        d_out = torch.from_numpy(rng.standard_normal((B, T, H, dv), dtype=np.float32)).to(dev)
        bwsb = R.bwd_workspace_bytes(B, T, H, dk, dv)
        bws = torch.empty(max(bwsb, 1), dtype=torch.uint8, device=dev)
        t0_, s0_ = sets[0][0], sets[0][1]
        tw = time.perf_counter()                 # warm-up: 50 ms of this call
        while time.perf_counter() - tw < 0.05:
            for _ in range(2):
                R.chunk_bwd(*t0_, d_out, initial_state=s0_, workspace=bws)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.bwd_steps):
            R.chunk_bwd(*t0_, d_out, initial_state=s0_, workspace=bws)
        e1.record(stream)
        torch.cuda.synchronize()
        bus = e0.elapsed_time(e1) * 1e3 / args.bwd_steps
        ntok = B * T * H
        bbytes = ntok * ((4 * dk + 2 * dv) * 2 + 4 * dv + (4 * dk + 2 * dv) * 4)
        backward = {"entry": "rodimus_ddts_chunk_bwd (state sweeps + chunk gradients)",
                    "workload": args.workload, "calls": args.bwd_steps,
                    "us_per_call": round(bus, 1), "tokens_per_s": round(B * T / (bus * 1e-6), 1),
                    "algorithmic_bytes_per_call": bbytes,
                    "algorithmic_GBps": round(bbytes / bus / 1e3, 1),
                    "frac_hbm": round(bbytes / bus / 1e3 / HBM_PEAK_GBPS, 4),
                    "workspace_bytes": bwsb}

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

    # ---------------- CPU baseline: the fp64 oracle on this host, same workload
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        # sample: the whole batch (all sequences and heads, whole length), in
        # repeated passes until about 10 s of CPU work have been timed
        Bs = B
        ins = [np.ascontiguousarray(x.f32(n)[:Bs]) for n in NAMES]
        s0 = None if x.initial_state is None else x.initial_state[:Bs]
        passes = 0
        c0 = time.perf_counter()
        ro = None
        while passes == 0 or time.perf_counter() - c0 < 10.0:
            o_, _ = oracle.fwd(*ins, s0, nthreads=nthreads)
            if ro is None:
                ro = o_
            passes += 1
        cs = time.perf_counter() - c0
        cpu = {"value": round(passes * Bs * T / cs, 1), "unit": "tokens/s",
               "cores": oracle.fwd.last_threads, "kind": "oracle",
               "sample": f"{Bs} of {B} sequences x {T} tokens x {H} heads of the same workload, "
                         f"{passes} passes, fp64 C oracle, {cs:.1f} s"}
        gpu_o = sets[0][2][:Bs].cpu().numpy()
        parity = {"max_abs_over_rms": oracle.rel_to_rms_error(gpu_o, ro), "bar": 1e-2,
                  "sample": "the CPU-baseline sample"}

    line = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "warmup_run": n_warm,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{args.workload}: B={B} T={T} H={H} dk={dk} dv={dv} "
                                   f"bf16 inputs, fp32 out/state, chunk {C}",
                       "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                       "rotating_input_sets": len(sets), "parallelism": "single GPU"},
            "roofline": roofline, "cpu_baseline": cpu, "other_forward": others or None,
            "decode": decode, "backward": backward, "serving": serving, "parity": parity}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
