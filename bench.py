#!/usr/bin/env python3
"""Throughput of the Q-Sparse decode hot path on one MI355X.

Default workload (the headline line): the Llama-7B-shaped squared-ReLU sparse
FFN at decode (d = 4096, ffn = 11008, bf16 weights, top-K 40% of the input
features, then top-K 40% of relu(u)^2 before the down projection), batch 1.
One step is one call of qs_sparse_ffn over one batch: the top-K of x and the
up projection over the selected rows of W_up^T with the squared-ReLU
epilogue, then the top-K of the intermediate and the down projection over
the rows of W_down^T it selects (at one token two launches, each selecting
inside its workgroups).  The weight rows are padded by 64 bf16 (--row-pad;
config.weight_row_pitch): with the natural pitches (multiples of 512 bytes)
the row segments of some column tiles share a subset of the memory channels
and those tiles finish last; the kernels read the same bytes either way.

Other workloads (--workload): c1 (fp32 1024x1024 linear, 8 tokens), c2g (the
same Llama-7B FFN with a gate: gated squared ReLU), c3
(int8 x ternary 4096x4096 linear), c4 (fused-QKV prefill through the MFMA
path, 2048 tokens), c4b (the same projection's training backward with the
straight-through estimator: dX and dW), c4s (the same prefill under Block
Q-Sparse 2:4 on the sparse matrix cores), c5 (Mistral-7B dReLU FFN decode),
c6 (Mixtral-47B-shaped dReLU MoE FFN decode: 8 experts, top-2).

Measurement:
  * inputs are resident in HBM before timing; weight copies rotate so that
    the footprint exceeds the 256 MB Infinity Cache where the weights are
    large, and eight activation batches rotate so the selections change;
  * the K timed steps are captured in one HIP graph (no host launch gaps)
    and timed with HIP events on the stream the library launches on;
  * roofline (c2): the step's weight-streaming kernels are timed alone,
    launch by launch in a graph, on the same inputs, through entry points
    that run exactly those kernels: at one token the up projection's column
    kernel (qs_sparse_linear for one bf16 token) and the down gather that
    selects h itself (qs_topk_gather_linear_acc), at more tokens the down
    gather (qs_gather_linear_acc, the accumulate form the step runs with
    fp32 outputs); the roofline is the longer (dominant) one, both are
    reported; achieved = algorithmic bytes (selected weight rows of the
    batch's union, each read once, plus activations and outputs) / time;
  * traffic: HBM bytes per launch from committed rocprofv3 PMC summaries
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), used
    only while the kernel source is unchanged since they were taken;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-linear tokens/s and HBM GB/s (% of roofline) at 7B FFN decode, 1 GPU"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_XROT = 8
C2_COPIES = 16    # relu2 FFN: 16 x 180 MB
C2G_COPIES = 8    # gated relu2 FFN: 8 x 271 MB (108 MB read per step at one token)
C5_COPIES = 6     # dReLU FFN: 6 x 352 MB (the whole gate, 117 MB, is read every step)
C6_COPIES = 3     # MoE: 3 x 2.8 GB (two experts' 361 MB per step)


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=480)
    p.add_argument("--warmup", type=int, default=48)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c2g", "c3", "c4", "c4b", "c4s", "c5", "c6"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--roofline-launches", type=int, default=96)
    p.add_argument("--row-pad", type=int, default=64,
                   help="bf16 columns of padding per W^T row: c2, c2g (all gathered matrices), c5 "
                        "(W_down^T); 0: natural rows")
    p.add_argument("--weight-copies", type=int, default=0,
                   help="weight copies to rotate over (0: the workload's default)")
    p.add_argument("--replays", type=int, default=50,
                   help="extra replays of the timed graph for the median per step")
    p.add_argument("--deterministic", action="store_true",
                   help="fixed-order split-K sums (qs_set_deterministic(1)) instead of float atomics")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 256 MiB device copy (for PMC byte calibration)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_graph(torch, stream, fn, steps, warmup, replays=0):
    """Warm up eagerly, capture `steps` calls of fn(i) in one HIP graph, time
    one replay bracketed by device synchronisations (the timed region of the
    JSON line).  With replays > 0 the same graph is then replayed that many
    more times, each replay between two events on the stream, and the
    per-replay times (ms) are returned as well."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn(i)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                fn(i)
        graph.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if replays <= 0:
            return ms
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
        ev[0].record(stream)
        for r in range(replays):
            graph.replay()
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
    return ms, [ev[r].elapsed_time(ev[r + 1]) for r in range(replays)]


def replay_stats(per_replay_ms, steps):
    """Median / min / max time per step over graph replays of `steps` steps."""
    import statistics
    per = [m * 1e3 / steps for m in per_replay_ms]
    return {"replays": len(per), "steps_per_replay": steps,
            "median_us_per_step": round(statistics.median(per), 3),
            "min_us_per_step": round(min(per), 3), "max_us_per_step": round(max(per), 3)}


def time_steps(args, torch, stream, fn, steps, warmup):
    """(ms per step of the timed region, replay statistics) for `steps` steps."""
    ms, per = time_graph(torch, stream, fn, steps, warmup, replays=args.replays)
    return ms / steps, replay_stats(per, steps)


# The sources a one-token FFN kernel is compiled from: the kernel file and the
# headers it includes, in this order.
GEMV_SOURCES = ("qs_gemv.hip", "qs_rowsel.h", "qs_select.h", "qs_internal.h")
# The one-token dReLU FFN's: its gate/up kernel's file, then the down gather's.
DRELU_SOURCES = ("qs_mfma.hip",) + GEMV_SOURCES


def sources_sha256(srcs=GEMV_SOURCES):
    """sha256 over the bytes of `srcs` (under csrc/), concatenated in order;
    None if one is missing."""
    h = hashlib.sha256()
    for f in srcs:
        path = os.path.join(ROOT, "sparse_activation_amd", "csrc", f)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def committed_traffic(name: str, row_pad: int, srcs=GEMV_SOURCES):
    """Traffic per launch from profiles/<name>, if it was counted on weight
    rows padded by `row_pad` elements and the hash of the sources it was
    counted on matches the current sources (else the kernel changed since)."""
    path = os.path.join(ROOT, "profiles", name)
    sha = sources_sha256(srcs)
    if sha is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m_pad = re.search(r"weight_row_pad:\s*([0-9]+)", text)
    if not m_pad or int(m_pad.group(1)) != row_pad:
        return None
    m_sha = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not (m_sha and m_val) or m_sha.group(1) != sha:
        return None
    return float(m_val.group(1))


def copy_calibration(torch, dev):
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 256 MiB device copies")


def probe_library():
    """qsprobe_stream_read from _lib/libqs_probe.so (a measurement probe built
    beside libqs.so, not part of its ABI)."""
    path = os.path.join(ROOT, "sparse_activation_amd", "_lib", "libqs_probe.so")
    fn = ctypes.CDLL(path).qsprobe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def bf16_dev(torch, np, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)


# ---------------------------------------------------------------- c2: relu2 FFN

def run_c2(args, torch, np, qs, datagen, dev, stream):
    B = args.batch
    log(f"workload c2: relu2 FFN decode B={B}; generating weights")
    c = datagen.c2_relu2_ffn(B)
    d, ffn = c["W_up"].shape[1], c["W_up"].shape[0]
    k_in, k_mid = c["K_in"], c["K_mid"]
    # Weight copies rotate so that the other steps' traffic between two visits
    # to one copy is several times the 256 MB Infinity Cache (MALL): a step
    # reads only the selected rows (72 MB at one token), so 16 copies put
    # 15 x 72 MB = 1.08 GB between visits.
    n_copies = args.weight_copies or C2_COPIES
    # The rows of W_up^T and W_down^T are padded by --row-pad bf16 (64: an odd
    # multiple of 128 bytes), so that no column tile's row segments sit at one
    # offset modulo 1 KiB on a subset of the memory channels; the kernels read
    # the same bytes.
    pad = args.row_pad
    wup0 = bf16_dev(torch, np, c["W_up"].T, dev)
    wdn0 = bf16_dev(torch, np, c["W_down"].T, dev)

    def padded_copy(src):
        base = torch.zeros((src.shape[0], src.shape[1] + pad), dtype=src.dtype, device=dev)
        base[:, :src.shape[1]] = src
        return base

    up_bases = [padded_copy(wup0) for _ in range(n_copies)]
    dn_bases = [padded_copy(wdn0) for _ in range(n_copies)]
    del wup0, wdn0
    wups = [b[:, :ffn] for b in up_bases]
    wdns = [b[:, :d] for b in dn_bases]
    xs = [bf16_dev(torch, np, datagen.c2_relu2_ffn(B, rotation=i, with_weights=False)["X"], dev)
          for i in range(N_XROT)]
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2, B, d, ffn),
                     dtype=torch.uint8, device=dev)

    def step(i):
        qs.qs_sparse_ffn(xs[i % N_XROT], qs.ACT_RELU2, k_in, k_mid, wups[i % n_copies],
                         wdns[i % n_copies], y=y, ws=ws)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    log(f"timed {args.steps} steps: {ms_step * 1e3:.2f} us/step, {B / (ms_step * 1e-3):.0f} tokens/s")

    # union sizes of the rotated batches (for the algorithmic bytes)
    u1, u2, hs = [], [], []
    for i in range(N_XROT):
        _, _, _, _, x1 = qs.qs_topk_mask(xs[i], k_in, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        _, h, _, _ = qs.qs_sparse_ffn(xs[i], qs.ACT_RELU2, k_in, k_mid, wups[0], wdns[0],
                                      want_h=True)
        _, _, _, _, x2 = qs.qs_topk_mask(h, k_mid, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        u1.append(x1)
        u2.append(x2)
        hs.append(h)
    torch.cuda.synchronize()
    un1 = [int((a != 0).any(0).sum()) for a in u1]
    un2 = [int((a != 0).any(0).sum()) for a in u2]

    def bytes_up(i):
        return un1[i] * ffn * 2 + B * d * 4 + B * ffn * 4

    def bytes_dn(i):
        return un2[i] * d * 2 + B * ffn * 4 + B * d * 4

    step_bytes = sum(bytes_up(i % N_XROT) + bytes_dn(i % N_XROT)
                     for i in range(args.steps)) / args.steps

    # roofline leg, launch by launch, each of the step's two weight-streaming
    # kernels in the form the step runs it, through an entry point that runs
    # that kernel alone (the same kernel, grid and bytes):
    #   * one token: the up projection's column kernel (qs_sparse_linear for
    #     one bf16 token; only the epilogue stores u instead of relu(u)^2),
    #     and the down gather that selects h itself
    #     (qs_topk_gather_linear_acc on the step's h);
    #   * more tokens: the down gather over the rows the descriptor selects
    #     (qs_gather_linear_acc on the sparsified h: the same rows in the same
    #     order), in the accumulate form unless fixed-order sums were asked for.
    # The roofline is the longer of the two (the dominant kernel); both are
    # reported.  Each figure is the median over graph replays of L launches,
    # divided by L: the average launch duration the kernel trace reports.
    L = args.roofline_launches
    ydn = torch.zeros((B, d), dtype=torch.float32, device=dev)
    kernels = {}

    def timed(name, fn, nbytes):
        _, per = time_graph(torch, stream, fn, L, 4, replays=args.replays)
        us = sorted(per)[len(per) // 2] * 1e3 / L
        gbps = nbytes / (us * 1e-6) / 1e9
        log(f"{name}: {us:.2f} us per launch, {gbps:.0f} GB/s")
        kernels[name] = {"us_per_launch": round(us, 3), "algorithmic_bytes_per_launch": round(nbytes),
                         "achieved_gbps": round(gbps, 1)}
        return us, gbps

    dn_bytes = sum(bytes_dn(i % N_XROT) for i in range(L)) / L
    up_bytes = sum(bytes_up(i % N_XROT) for i in range(L)) / L
    if B == 1 and not args.deterministic:
        def down_launch(i):
            qs.qs_topk_gather_linear_acc(hs[i % N_XROT], k_mid, wdns[i % n_copies], ydn)
        dn_name = "gather_sel_kernel (down, selection of h inside)"
    else:
        ws_dn = qs.gather_workspace(B, ffn, d, dev)
        gather = qs.qs_gather_linear if args.deterministic else qs.qs_gather_linear_acc

        def down_launch(i):
            gather(u2[i % N_XROT], wdns[i % n_copies], y=ydn, ws=ws_dn)
        # bf16 W_down^T: token tiles of 5-16 rows run the bf16 MFMA gather.
        dn_name = "gather_bmfma_kernel (down)" if B > 4 else "gather_gemv_kernel (down)"
    cands = [(dn_name,) + timed(dn_name, down_launch, dn_bytes) + (dn_bytes,)]
    if B == 1:
        yup = torch.empty((B, ffn), dtype=torch.float32, device=dev)
        ws_lin = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR, B, d, ffn),
                             dtype=torch.uint8, device=dev)

        def up_launch(i):
            qs.qs_sparse_linear(xs[i % N_XROT], k_in, wups[i % n_copies], y=yup, ws=ws_lin)

        up_name = "up_cols_kernel (up, selection of x inside)"
        cands.append((up_name,) + timed(up_name, up_launch, up_bytes) + (up_bytes,))
    dom, us_launch, achieved, bytes_launch = max(cands, key=lambda c: c[1])
    traffic = None
    if dom.startswith("up_cols"):
        traffic = committed_traffic("up_cols_llama7b_relu2_b1_traffic.md", pad)
    elif dom.startswith("gather_sel"):
        traffic = committed_traffic("gather_sel_llama7b_relu2_b1_traffic.md", pad)
    elif dom.startswith("gather_gemv") and not args.deterministic:
        traffic = committed_traffic(f"gather_gemv_llama7b_relu2_b{B}_traffic.md", pad)
    elif dom.startswith("gather_bmfma") and not args.deterministic:
        traffic = committed_traffic(f"gather_bmfma_down_llama7b_relu2_b{B}_traffic.md", pad)
    dom = dom.split(" ")[0]

    # ceiling reference: a plain streaming read of the same bytes per launch,
    # rotating over chunks of the weight copies (> 256 MB, so not from the MALL)
    flat = [t.view(-1).view(torch.uint8) for t in up_bases + dn_bases]
    nb = min(int(bytes_launch), min(f.numel() for f in flat)) // 16 * 16
    chunks = [f[o:o + nb] for f in flat for o in range(0, f.numel() - nb + 1, nb)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream_read = probe_library()

    def probe(i):
        rc = stream_read(ctypes.c_void_p(chunks[i % len(chunks)].data_ptr()), nb,
                         ctypes.c_void_p(sink.data_ptr()),
                         ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        if rc != 0:
            raise RuntimeError(f"stream-read probe failed ({rc})")

    _, per = time_graph(torch, stream, probe, L, 4, replays=max(5, args.replays // 5))
    ms_probe = sorted(per)[len(per) // 2]
    probe_gbps = nb * L / (ms_probe * 1e-3) / 1e9
    log(f"stream-read probe, {nb / 1e6:.1f} MB per launch over {len(chunks)} chunks: "
        f"{probe_gbps:.0f} GB/s; {dom} at {achieved / probe_gbps:.1%} of it")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_c2(c, args.cpu_seconds)
    return {
        "metric": METRIC, "value": round(B / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(ms_step, 6), "dtype": "bf16",
        "config": {"workload": "llama7b_relu2_ffn_decode", "batch": B, "d": d, "ffn": ffn,
                   "k_in": k_in, "k_mid": k_mid, "weights": "bf16",
                   "weight_row_pad": pad, "weight_row_pitch": {"w_up_t": ffn + pad, "w_down_t": d + pad},
                   "weight_copies": n_copies, "x_rotations": N_XROT},
        "hbm_gbps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "union_rows_up": un1, "union_rows_down": un2,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": dom,
                     "algorithmic_bytes_per_launch": round(bytes_launch),
                     "us_per_launch": round(us_launch, 3),
                     "stream_read_probe_gbps": round(probe_gbps, 1),
                     "frac_of_stream_read_probe": round(achieved / probe_gbps, 4),
                     "kernels": kernels},
        "timing": timing, "cpu_baseline": cpu,
    }


def host_info():
    """Threads the oracle may use on this host (the CPU affinity set, capped by
    OMP_NUM_THREADS where the environment sets one), the CPU model and the
    BLAS library NumPy was built with."""
    import numpy as np
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{dep.get('name', '?')} {dep.get('version', '')}".strip()
    except Exception:
        pass
    return threads, model, blas


def cpu_baseline_c2(c, seconds):
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import datagen
    import oracle
    threads, model, blas = host_info()
    w_up = c["W_up"].astype(np.float64)
    w_dn = c["W_down"].astype(np.float64)
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
        times, n, t0 = [], 0, time.perf_counter()
        while n < 4096:   # bounded by --cpu-seconds of oracle time
            x = datagen.c2_relu2_ffn(1, rotation=n % N_XROT, with_weights=False)["X"]
            t1 = time.perf_counter()
            oracle.ffn_relu2(x, c["K_in"], w_up, c["K_mid"], w_dn)
            times.append(time.perf_counter() - t1)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = sum(times)
    med = sorted(times)[len(times) // 2]
    log(f"cpu oracle: {n} tokens in {dt:.1f} s ({used} BLAS threads, {model}, {blas})")
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "median_ms_per_token": round(med * 1e3, 2), "cpu_model": model, "blas": blas,
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} single-token steps of the same workload (B=1), float64 NumPy "
                      f"oracle (select, matmuls, epilogues; input generation not timed)"}


# ---------------------------------------------------------------- other workloads

def run_c5(args, torch, np, qs, datagen, dev, stream):
    B = args.batch
    log(f"workload c5: dReLU FFN decode B={B}; generating weights")
    c = datagen.c5_drelu_ffn(B)
    ffn, d = c["W_gate"].shape
    n_copies = args.weight_copies or C5_COPIES                           # 5 x >= 166 MB between visits
    wg = [bf16_dev(torch, np, c["W_gate"], dev)]
    wu = [bf16_dev(torch, np, c["W_up"], dev)]
    for _ in range(n_copies - 1):
        wg.append(wg[0].clone()); wu.append(wu[0].clone())
    # W_down^T rows padded by --row-pad bf16 (the down gather's column tiles,
    # as in c2); W_gate and W_up are read in whole rows and keep theirs.
    pad = args.row_pad
    wd0 = bf16_dev(torch, np, c["W_down"].T, dev)
    wd = []
    for _ in range(n_copies):
        base = torch.zeros((ffn, d + pad), dtype=wd0.dtype, device=dev)
        base[:, :d] = wd0
        wd.append(base[:, :d])
    del wd0
    bg = torch.from_numpy(c["b_gate"]).to(dev)
    bu = torch.from_numpy(c["b_up"]).to(dev)
    xs = [bf16_dev(torch, np, datagen.c5_drelu_ffn(B, rotation=i, with_weights=False)["X"], dev)
          for i in range(N_XROT)]
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_DRELU, B, d, ffn),
                     dtype=torch.uint8, device=dev)

    def step(i):
        j = i % n_copies
        qs.qs_sparse_ffn(xs[i % N_XROT], qs.ACT_DRELU, d, -1, wu[j], wd[j], w_gate=wg[j],
                         b_gate=bg, b_up=bu, y=y, ws=ws)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    # measured unions: gate read in full, up rows with g > 0 for some token, down rows with h != 0
    hs = [qs.qs_sparse_ffn(xs[i], qs.ACT_DRELU, d, -1, wu[0], wd[0], w_gate=wg[0], b_gate=bg,
                           b_up=bu, want_h=True)[1] for i in range(N_XROT)]
    g_pos = []
    for i in range(N_XROT):
        g = xs[i].float() @ wg[0].float().t() + bg
        g_pos.append(int((g > 0).any(0).sum()))
    nz = [int((h != 0).any(0).sum()) for h in hs]
    zero_frac = float(np.mean([float((h == 0).float().mean()) for h in hs]))
    rb = d * 2
    step_bytes = np.mean([ffn * rb + g_pos[i] * rb + nz[i] * rb for i in range(N_XROT)])
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"c5: {ms_step * 1e3:.2f} us/step, {achieved:.0f} GB/s, zero fraction of h {zero_frac:.3f}")
    return {
        "metric": "dReLU sparse FFN tokens/s at Mistral-7B decode, 1 GPU", "unit": "tokens/s",
        "value": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 6), "dtype": "bf16",
        "config": {"workload": "mistral7b_drelu_ffn_decode", "batch": B, "d": d, "ffn": ffn,
                   "w_down_t_row_pad": pad,
                   "weight_copies": n_copies, "x_rotations": N_XROT,
                   "zero_fraction_h": round(zero_frac, 4), "up_rows_read": g_pos,
                   "down_rows_read": nz},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic("mistral7b_drelu_ffn_b1_step_traffic.md", pad,
                                                  DRELU_SOURCES)
                     if B == 1 and not args.deterministic else None,
                     "kernel": "whole FFN step (gate/up + down)",
                     "algorithmic_bytes_per_step": round(float(step_bytes))},
        "timing": timing, "cpu_baseline": None,
    }


def run_c4(args, torch, np, qs, datagen, dev, stream):
    log("workload c4: fused-QKV prefill through the MFMA path")
    c = datagen.c4_prefill_qkv()
    (m, kdim), n = c["X"].shape, c["W"].shape[0]
    w = bf16_dev(torch, np, c["W"], dev)
    xs = [bf16_dev(torch, np, datagen.c4_prefill_qkv(rotation=i, with_weights=False)["X"], dev)
          for i in range(2)]
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR, m, kdim, n), dtype=torch.uint8,
                     device=dev)

    def step(i):
        qs.qs_sparse_linear(xs[i % 2], c["K"], w, layout=qs.LAYOUT_W, y=y, ws=ws)

    steps = max(4, min(args.steps, 40))
    ms_step, timing = time_steps(args, torch, stream, step, steps, 4)
    flops = 2.0 * m * n * kdim
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"c4: {ms_step * 1e3:.1f} us/step, {tflops:.0f} TFLOP/s (top-K + GEMM)")
    return {
        "metric": "masked-MFMA prefill tokens/s (fused QKV 4096->12288), 1 GPU", "unit": "tokens/s",
        "value": round(m / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 6), "dtype": "bf16",
        "steps": steps,
        "config": {"workload": "qkv_prefill_2048x4096x12288", "tokens": m, "d": kdim, "n": n,
                   "k": c["K"]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "whole call (top-K + gemm_bf16_deep_kernel)"},
        "timing": timing, "cpu_baseline": None,
    }


def run_c6(args, torch, np, qs, datagen, dev, stream):
    B = args.batch
    log(f"workload c6: Mixtral-47B-shaped dReLU MoE FFN decode B={B}; generating weights")
    c = datagen.c6_moe_drelu_ffn(B)
    n_exp, ffn, d = c["W_gate"].shape
    top_k = 2
    bf = torch.bfloat16
    wr = bf16_dev(torch, np, c["W_router"], dev)
    mats = {}
    for name in ("W_gate", "W_up", "W_down_t"):      # expert by expert: bounded host copies
        t = torch.empty((n_exp, ffn, d), dtype=bf, device=dev)
        for e in range(n_exp):
            t[e] = torch.from_numpy(c[name][e]).to(dev).to(bf)
        mats[name] = t
        c[name] = None
    bg = torch.from_numpy(c["b_gate"]).to(dev)
    bu = torch.from_numpy(c["b_up"]).to(dev)
    xs = [bf16_dev(torch, np, datagen.c6_moe_drelu_ffn(B, rotation=i, with_weights=False)["X"], dev)
          for i in range(8)]
    y = torch.empty((B, d), dtype=bf, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_MOE_FFN, B * top_k, d, ffn),
                     dtype=torch.uint8, device=dev)

    # Algorithmic bytes of each input batch (bookkeeping outside the timed
    # region): per expert the batch uses, its whole gate matrix, the up rows
    # whose gate is positive for a token routed to it, the down rows where h is
    # nonzero for such a token; plus the router, x and y.
    step_bytes, up_frac, down_frac = [], [], []
    for i in range(8):
        _, _, ex, _, h = qs.qs_sparse_moe_ffn(xs[i], top_k, wr, mats["W_gate"], mats["W_up"],
                                              mats["W_down_t"], bg, bu, want_all=True)
        rows_read = 0
        for e in sorted(set(ex.flatten().tolist())):
            sel = ex == e                                  # [B, top_k]
            toks = sel.any(dim=1).nonzero().flatten()
            g = xs[i][toks].float() @ mats["W_gate"][e].float().t() + bg[e]
            up = int((g > 0).any(dim=0).sum())
            down = int((h[sel] != 0).any(dim=0).sum())
            rows_read += ffn + up + down
            up_frac.append(up / ffn)
            down_frac.append(down / ffn)
        step_bytes.append(rows_read * d * 2 + n_exp * d * 2 + 2 * B * d * 2)
    torch.cuda.synchronize()

    # Copies of the expert weights rotate as well, so that an expert two
    # consecutive batches both route to is not re-read from the MALL.
    n_copies = args.weight_copies or C6_COPIES
    copies = [(mats["W_gate"], mats["W_up"], mats["W_down_t"])]
    for _ in range(n_copies - 1):
        copies.append(tuple(t.clone() for t in copies[0]))

    def step(i):
        g, u, dn = copies[i % n_copies]
        qs.qs_sparse_moe_ffn(xs[i % 8], top_k, wr, g, u, dn, bg, bu, y=y, ws=ws)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    alg = float(np.mean(step_bytes))
    achieved = alg / (ms_step * 1e-3) / 1e9
    log(f"c6: {ms_step * 1e3:.2f} us/step, {B / (ms_step * 1e-3):.0f} tokens/s, "
        f"{achieved:.0f} GB/s on {alg / 1e6:.1f} MB; up rows {np.mean(up_frac):.3f}, "
        f"down rows {np.mean(down_frac):.3f} of each used expert")
    return {
        "metric": "dReLU MoE FFN tokens/s at Mixtral-47B decode (8 experts, top-2), 1 GPU",
        "unit": "tokens/s", "value": round(B / (ms_step * 1e-3), 1),
        "ms_per_step": round(ms_step, 6), "dtype": "bf16",
        "config": {"workload": "mixtral47b_drelu_moe_ffn_decode", "batch": B, "d": d, "ffn": ffn,
                   "experts": n_exp, "top_k": top_k, "x_rotations": 8,
                   "weight_copies": n_copies,
                   "up_rows_frac": round(float(np.mean(up_frac)), 4),
                   "down_rows_frac": round(float(np.mean(down_frac)), 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "whole MoE step (router, gate/up, down gather, combine)",
                     "algorithmic_bytes_per_step": int(alg)},
        "timing": timing, "cpu_baseline": None,
    }


def run_c4s(args, torch, np, qs, datagen, dev, stream):
    log("workload c4s: fused-QKV prefill under Block Q-Sparse (2:4) on sparse MFMA")
    c = datagen.c4_prefill_qkv()
    (m, kdim), n = c["X"].shape, c["W"].shape[0]
    w = bf16_dev(torch, np, c["W"], dev)
    xs = [bf16_dev(torch, np, datagen.c4_prefill_qkv(rotation=i, with_weights=False)["X"], dev)
          for i in range(2)]
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_BLOCK_SPARSE_LINEAR, m, kdim, n),
                     dtype=torch.uint8, device=dev)

    def step(i):
        qs.qs_block_sparse_linear(xs[i % 2], w, y=y, ws=ws)

    steps = max(4, min(args.steps, 40))
    ms_step, timing = time_steps(args, torch, stream, step, steps, 4)
    kept_flops = 2.0 * m * n * (kdim // 2)            # the MACs on kept entries
    tflops = kept_flops / (ms_step * 1e-3) / 1e12
    dense_eq = 2 * tflops
    log(f"c4s: {ms_step * 1e3:.1f} us/step, {tflops:.0f} TFLOP/s on kept entries "
        f"({dense_eq:.0f} dense-equivalent), pack + sparse GEMM")
    return {
        "metric": "Block Q-Sparse (2:4) prefill tokens/s (fused QKV 4096->12288), 1 GPU",
        "unit": "tokens/s", "value": round(m / (ms_step * 1e-3), 1),
        "ms_per_step": round(ms_step, 6), "dtype": "bf16", "steps": steps,
        "config": {"workload": "qkv_prefill_block24_2048x4096x12288", "tokens": m, "d": kdim,
                   "n": n, "pattern": "2:4"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "dense_equivalent_tflops": round(dense_eq, 1),
                     "kernel": "whole call (nm24_pack_kernel + gemm_sp24_kernel)"},
        "timing": timing, "cpu_baseline": None,
    }


def run_c4b(args, torch, np, qs, datagen, dev, stream):
    log("workload c4b: fused-QKV training backward (straight-through estimator)")
    c = datagen.c4_prefill_qkv()
    (m, kdim), n = c["X"].shape, c["W"].shape[0]
    w = bf16_dev(torch, np, c["W"], dev)
    xs = [bf16_dev(torch, np, datagen.c4_prefill_qkv(rotation=i, with_weights=False)["X"], dev)
          for i in range(2)]
    gys = [bf16_dev(torch, np, datagen.c4_backward_grad(m, n, rotation=i), dev) for i in range(2)]
    dx = torch.empty((m, kdim), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((n, kdim), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR_BACKWARD, m, kdim, n),
                     dtype=torch.uint8, device=dev)

    def step(i, want_dx=True, want_dw=True):
        qs.qs_sparse_linear_backward(xs[i % 2], c["K"], w, gys[i % 2], layout=qs.LAYOUT_W,
                                     want_dx=want_dx, want_dw=want_dw, dx=dx, dw=dw, ws=ws)

    steps = max(4, min(args.steps, 40))
    ms_step, timing = time_steps(args, torch, stream, step, steps, 4)
    ms_dx = time_graph(torch, stream, lambda i: step(i, want_dw=False), steps, 2) / steps
    ms_dw = time_graph(torch, stream, lambda i: step(i, want_dx=False), steps, 2) / steps
    flops = 2.0 * m * n * kdim
    tflops = 2 * flops / (ms_step * 1e-3) / 1e12
    log(f"c4b: {ms_step * 1e3:.1f} us/step, {tflops:.0f} TFLOP/s (top-K + dW GEMM + dX GEMM); "
        f"dX alone {ms_dx * 1e3:.1f} us = {flops / (ms_dx * 1e-3) / 1e12:.0f} TFLOP/s, "
        f"dW with its top-K {ms_dw * 1e3:.1f} us = {flops / (ms_dw * 1e-3) / 1e12:.0f} TFLOP/s")
    return {
        "metric": "STE backward tokens/s (fused QKV 4096->12288: dX and dW), 1 GPU",
        "unit": "tokens/s", "value": round(m / (ms_step * 1e-3), 1),
        "ms_per_step": round(ms_step, 6), "dtype": "bf16", "steps": steps,
        "config": {"workload": "qkv_backward_2048x4096x12288", "tokens": m, "d": kdim, "n": n,
                   "k": c["K"], "dx": "bf16", "dw": "fp32"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "kernel": "whole call (top-K + two gemm_bf16_deep_kernel launches)",
                     "dx_us": round(ms_dx * 1e3, 2), "dw_us_with_topk": round(ms_dw * 1e3, 2)},
        "timing": timing, "cpu_baseline": None,
    }


def run_c2g(args, torch, np, qs, datagen, dev, stream):
    B = args.batch
    log(f"workload c2g: gated relu2 FFN decode B={B}; generating weights")
    c = datagen.c2g_relu2glu_ffn(B)
    d, ffn = c["W_up"].shape[1], c["W_up"].shape[0]
    k_in, k_mid = c["K_in"], c["K_mid"]
    n_copies = args.weight_copies or C2G_COPIES                          # 7 x >= 108 MB between visits
    pad = args.row_pad   # padded rows, as in c2

    def copies(a):
        src = bf16_dev(torch, np, a, dev)
        out = []
        for _ in range(n_copies):
            base = torch.zeros((src.shape[0], src.shape[1] + pad), dtype=src.dtype, device=dev)
            base[:, :src.shape[1]] = src
            out.append(base[:, :src.shape[1]])
        return out

    wg, wu, wd = copies(c["W_gate"].T), copies(c["W_up"].T), copies(c["W_down"].T)
    xs = [bf16_dev(torch, np, datagen.c2g_relu2glu_ffn(B, rotation=i, with_weights=False)["X"], dev)
          for i in range(N_XROT)]
    y = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_FFN_RELU2_GLU, B, d, ffn),
                     dtype=torch.uint8, device=dev)

    def step(i):
        j = i % n_copies
        qs.qs_sparse_ffn(xs[i % N_XROT], qs.ACT_RELU2_GLU, k_in, k_mid, wu[j], wd[j],
                         w_gate=wg[j], y=y, ws=ws)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    # measured unions: rows of W_gate^T and W_up^T selected by some token, rows of W_down^T
    u1, u2, hs = [], [], []
    for i in range(N_XROT):
        _, _, _, _, x1 = qs.qs_topk_mask(xs[i], k_in, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        _, h, _, _ = qs.qs_sparse_ffn(xs[i], qs.ACT_RELU2_GLU, k_in, k_mid, wu[0], wd[0],
                                      w_gate=wg[0], want_h=True)
        _, _, _, _, x2 = qs.qs_topk_mask(h, k_mid, want_mask=False, want_idx=False,
                                          want_desc=False, want_xs=True)
        u1.append(int((x1 != 0).any(0).sum()))
        u2.append(int((x2 != 0).any(0).sum()))
    step_bytes = np.mean([2 * u1[i] * ffn * 2 + u2[i] * d * 2 + B * (d * 4 * 2 + ffn * 4 * 3)
                          for i in range(N_XROT)])
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"c2g: {ms_step * 1e3:.2f} us/step, {B / (ms_step * 1e-3):.0f} tokens/s, {achieved:.0f} GB/s")
    return {
        "metric": "gated squared-ReLU sparse FFN tokens/s at Llama-7B decode, 1 GPU",
        "unit": "tokens/s", "value": round(B / (ms_step * 1e-3), 1),
        "ms_per_step": round(ms_step, 6), "dtype": "bf16",
        "config": {"workload": "llama7b_relu2glu_ffn_decode", "batch": B, "d": d, "ffn": ffn,
                   "k_in": k_in, "k_mid": k_mid, "weight_row_pad": pad, "weight_copies": n_copies,
                   "x_rotations": N_XROT, "union_rows_in": u1, "union_rows_mid": u2},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic("llama7b_relu2glu_ffn_b1_step_traffic.md", pad)
                     if B == 1 and not args.deterministic else None,
                     "kernel": "whole FFN step (gate, up, top-K of h, down)",
                     "algorithmic_bytes_per_step": round(float(step_bytes))},
        "timing": timing, "cpu_baseline": None,
    }


def run_c3(args, torch, np, qs, datagen, dev, stream):
    B = args.batch
    log(f"workload c3: int8 x ternary linear B={B}")
    c = datagen.c3_i8t_linear(B)
    t, alpha = qs.qs_ternarize(c["W"])
    n, d = c["W"].shape
    packed = torch.from_numpy(qs.qs_pack_ternary(t)).to(dev)
    copies = [packed] + [packed.clone() for _ in range(127)]   # 128 x 4 MB > 256 MB MALL
    xs = [torch.from_numpy(datagen.c3_i8t_linear(B, rotation=i, with_weights=False)["X"]).to(dev)
          for i in range(N_XROT)]
    acc = torch.empty((B, n), dtype=torch.int32, device=dev)
    y = torch.empty((B, n), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR_I8T, B, d, n), dtype=torch.uint8,
                     device=dev)

    def step(i):
        qs.qs_sparse_linear_i8t(xs[i % N_XROT], c["K"], copies[i % 128], alpha, n, acc=acc, y=y,
                                ws=ws, want_all=False)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    log(f"c3: {ms_step * 1e3:.2f} us/step")
    return {
        "metric": "int8 x ternary sparse linear tokens/s (4096x4096), 1 GPU", "unit": "tokens/s",
        "value": round(B / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 6), "dtype": "int8",
        "config": {"workload": "bitnet_i8t_linear_4096", "batch": B, "k": c["K"]},
        "roofline": None, "timing": timing, "cpu_baseline": None,
    }


def run_c1(args, torch, np, qs, datagen, dev, stream):
    log("workload c1: fp32 linear [8,1024] x [1024,1024]")
    c = datagen.c1_linear()
    wt = torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)
    copies = [wt] + [wt.clone() for _ in range(127)]
    xs = [torch.from_numpy(datagen.c1_linear(rotation=i, with_weights=False)["X"]).to(dev)
          for i in range(N_XROT)]
    y = torch.empty((8, 1024), dtype=torch.float32, device=dev)
    ws = torch.empty(qs.qs_workspace_bytes(qs.OP_SPARSE_LINEAR, 8, 1024, 1024), dtype=torch.uint8,
                     device=dev)

    def step(i):
        qs.qs_sparse_linear(xs[i % N_XROT], c["K"], copies[i % 128], y=y, ws=ws)

    ms_step, timing = time_steps(args, torch, stream, step, args.steps, args.warmup)
    log(f"c1: {ms_step * 1e3:.2f} us/step")
    return {
        "metric": "fp32 sparse linear tokens/s (1024x1024, 8 tokens), 1 GPU", "unit": "tokens/s",
        "value": round(8 / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 6), "dtype": "f32",
        "config": {"workload": "fp32_linear_1024", "batch": 8, "k": c["K"]},
        "roofline": None, "timing": timing, "cpu_baseline": None,
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import datagen
    import sparse_activation_amd as qs

    qs.load()
    qs.qs_set_deterministic(args.deterministic)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    if args.copy_calibration:
        copy_calibration(torch, dev)
    run = {"c1": run_c1, "c2": run_c2, "c2g": run_c2g, "c3": run_c3, "c4": run_c4, "c4b": run_c4b, "c4s": run_c4s, "c6": run_c6,
           "c5": run_c5}[args.workload]
    out = run(args, torch, np, qs, datagen, dev, stream)
    line = {"metric": out.pop("metric"), "value": out.pop("value"), "unit": out.pop("unit"),
            "n_gpus": 1, "steps": out.pop("steps", args.steps), "warmup": args.warmup,
            "ms_per_step": out.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": out.pop("dtype"),
            "data": "synthetic (seeded Student-t(4) activations, N(0,0.02) weights)"}
    line.update(out)
    if isinstance(line.get("config"), dict):
        line["config"]["split_k_sums"] = "fixed_order" if args.deterministic else "atomic"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
