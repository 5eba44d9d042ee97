#!/usr/bin/env python3
"""Throughput of the Q-Sparse decode hot path on one MI355X.

Default workload: the Llama-7B-shaped squared-ReLU sparse FFN at decode
(d = 4096, ffn = 11008, bf16 weights, top-K 40% of the input features, then
top-K 40% of relu(u)^2 before the down projection).  One step is one call of
qs_sparse_ffn over one batch: top-K of x, gathered up projection with the
squared-ReLU epilogue, top-K of the intermediate, gathered down projection.

Measurement:
  * inputs are resident in HBM before timing; three copies of the weights
    (541 MB, more than the 256 MB Infinity Cache) and eight activation batches
    rotate from step to step, so the selected rows change and are not served
    from the cache;
  * the K timed steps are captured in one HIP graph (no host launch gaps)
    and timed with HIP events on the stream the library launches on;
  * roofline: the gather GEMV (the dominant kernel) is timed alone, launch by
    launch in a graph, on the same inputs; achieved = algorithmic bytes
    (selected weight rows of the batch's union, each read once, plus its
    activations and outputs) / measured time, against 8 TB/s;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-linear tokens/s and HBM GB/s (% of roofline) at 7B FFN decode, 1 GPU"
HBM_PEAK_GBPS = 8000.0
N_WCOPIES = 3
N_XROT = 8


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--roofline-launches", type=int, default=96)
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import datagen
    import sparse_activation_amd as qs

    qs.load()
    dev = torch.device("cuda:0")
    B = args.batch
    log(f"workload: relu2 FFN decode B={B}; generating weights")
    c = datagen.c2_relu2_ffn(B)
    d, ffn = c["W_up"].shape[1], c["W_up"].shape[0]
    k_in, k_mid = c["K_in"], c["K_mid"]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)

    wup0 = bf16(c["W_up"].T)          # W_up^T   [d, ffn]
    wdn0 = bf16(c["W_down"].T)        # W_down^T [ffn, d]
    wups = [wup0] + [wup0.clone() for _ in range(N_WCOPIES - 1)]
    wdns = [wdn0] + [wdn0.clone() for _ in range(N_WCOPIES - 1)]
    xs = [bf16(datagen.c2_relu2_ffn(B, rotation=i, with_weights=False)["X"])
          for i in range(N_XROT)]
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2, B, d, ffn),
                     dtype=torch.uint8, device=dev)

    def step(i):
        qs.qs_sparse_ffn(xs[i % N_XROT], qs.ACT_RELU2, k_in, k_mid, wups[i % N_WCOPIES],
                         wdns[i % N_WCOPIES], y=y, ws=ws)

    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        log(f"warmup {args.warmup} steps")
        for i in range(args.warmup):
            step(i)
        stream.synchronize()
        log(f"capturing {args.steps} steps in a graph")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                step(i)
        graph.replay()                       # untimed replay (first-touch of the graph)
        stream.synchronize()

        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    tokens_per_s = B / (ms_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step, {tokens_per_s:.0f} tokens/s")

    # ---- union sizes of the rotated batches (for the algorithmic bytes)
    u1, u2 = [], []
    for i in range(N_XROT):
        _, _, _, _, x1 = qs.qs_topk_mask(xs[i], k_in, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        _, h, _, _ = qs.qs_sparse_ffn(xs[i], qs.ACT_RELU2, k_in, k_mid, wups[0], wdns[0],
                                      want_h=True)
        _, _, _, _, x2 = qs.qs_topk_mask(h, k_mid, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        u1.append(x1)
        u2.append(x2)
    torch.cuda.synchronize(dev)
    un1 = [int((a != 0).any(0).sum()) for a in u1]
    un2 = [int((a != 0).any(0).sum()) for a in u2]

    def bytes_up(i):
        return un1[i] * ffn * 2 + B * d * 4 + B * ffn * 4

    def bytes_dn(i):
        return un2[i] * d * 2 + B * ffn * 4 + B * d * 4

    step_bytes = sum(bytes_up(i % N_XROT) + bytes_dn(i % N_XROT)
                     for i in range(args.steps)) / args.steps

    # ---- roofline leg: the gather GEMV alone, launch by launch
    L = args.roofline_launches
    yup = torch.empty((B, ffn), dtype=torch.float32, device=dev)
    ydn = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws_up = qs.gather_workspace(B, d, ffn, dev)
    ws_dn = qs.gather_workspace(B, ffn, d, dev)
    torch.cuda.synchronize(dev)
    with torch.cuda.stream(stream):
        for i in range(4):
            qs.qs_gather_linear(u1[i % N_XROT], wups[i % N_WCOPIES], y=yup, ws=ws_up)
            qs.qs_gather_linear(u2[i % N_XROT], wdns[i % N_WCOPIES], y=ydn, ws=ws_dn)
        stream.synchronize()
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=stream):
            for i in range(L):
                qs.qs_gather_linear(u1[i % N_XROT], wups[i % N_WCOPIES], y=yup, ws=ws_up)
                qs.qs_gather_linear(u2[i % N_XROT], wdns[i % N_WCOPIES], y=ydn, ws=ws_dn)
        g2.replay()
        stream.synchronize()
        torch.cuda.synchronize(dev)
        e0.record(stream)
        g2.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms_gemv = e0.elapsed_time(e1)
    gemv_bytes = sum(bytes_up(i % N_XROT) + bytes_dn(i % N_XROT) for i in range(L))
    us_launch = ms_gemv * 1e3 / (2 * L)
    achieved = gemv_bytes / (ms_gemv * 1e-3) / 1e9
    log(f"gather GEMV: {us_launch:.2f} us per launch (avg of up and down), {achieved:.0f} GB/s")

    # ---- CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Student-t(4) activations, N(0,0.02) weights; datagen recipe)",
        "config": {"workload": "llama7b_relu2_ffn_decode", "batch": B, "d": d, "ffn": ffn,
                   "k_in": k_in, "k_mid": k_mid, "weights": "bf16",
                   "weight_copies": N_WCOPIES, "x_rotations": N_XROT},
        "hbm_gbps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "union_rows_up": un1,
        "union_rows_down": un2,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "gather_gemv_kernel",
                     "us_per_launch": round(us_launch, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(c, seconds):
    import numpy as np

    import datagen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    w_up = c["W_up"].astype(np.float64)
    w_dn = c["W_down"].astype(np.float64)
    n, t0 = 0, time.perf_counter()
    while n < 64:
        x = datagen.c2_relu2_ffn(1, rotation=n % N_XROT, with_weights=False)["X"]
        oracle.ffn_relu2(x, c["K_in"], w_up, c["K_mid"], w_dn)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    log(f"cpu oracle: {n} tokens in {dt:.1f} s")
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} single-token steps of the same workload (B=1), float64 NumPy oracle"}


if __name__ == "__main__":
    main()
