#!/usr/bin/env python3
"""Throughput of the KLA forward scan on one MI355X.

Workload lm45m_bf16: B=8, H=8, T=2048, d_k=d_v=64, bf16 inputs, fp32 scan,
seeded synthetic inputs (kla_inputs recipe).  One step = one kla_forward call
over the whole batch (precision scan, gates, chunked mean recursion, readout).
Inputs are resident in HBM before timing; three input/output copies rotate so
the 256 MB last-level cache cannot hold the working set between steps.

Timed K steps: after the warm-up, K eager calls with a HIP event pair around
each (per-launch min and max), then the same K steps captured once in a HIP
graph and replayed (wall clock and one event pair around the replay).

Prints one JSON line:
  value      tokens/s (B*H*T per step / wall time per step of the graph-launched
             K steps; `launch` reports the eager loop's figure beside it)
  roofline   dominant kernel (kla_fwd_run_kernel, the run-streaming forward): algorithmic bytes
             per launch / mean launch duration (HIP events on the launch
             stream around the replayed K launches), against the 8 TB/s HBM
             peak, with a measured device-copy bandwidth as second
             denominator; traffic = measured HBM bytes per launch from
             committed counter profiles when they were taken on the current
             kernel sources, else null
  cpu_baseline  the float64 oracle on the host, timed on the same workload
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

METRIC = "KLA fwd tokens/s (B*H*T) at dk=dv=64,T=2048; % of HBM roofline"
WORKLOAD = "lm45m_bf16"
PEAK_HBM_GBS = 8000.0
KERNEL = "kla_fwd_run_kernel"  # the run-streaming forward (bf16, d_k = d_v = 64)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kla_fwd_lm45m_bf16_traffic.json")
SOURCES = ["kla_forward_run.hip", "kla_device.h", "kla_internal.h"]
PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of the MI355X (no sparsity)
NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


def algorithmic_bytes(B, H, T, dk, dv, esz):
    """Bytes the method must move: per token q, k, log_decay, proc_noise,
    val_prec (d_k each) and v (d_v) read, y (d_v) written; per head the fp32
    state in (lambda0, M0) and out (lambda_T, M_T)."""
    per_token = (5 * dk + dv) * esz + dv * esz
    state = B * H * (dk + dk * dv) * 4 * 2
    return B * H * T * per_token + state


def run_plan(nheads, T, ncu):
    """Runs per head and their tile counts as the library plans them for the
    run-streaming kernel (kla_forward_run.hip, fwd_run_plan): the run count
    that minimises rounds of workgroups x (tiles per workgroup + 4, a run's
    start and end), fewest runs on ties, the tiles split as evenly as they
    go.  Returns the list of tile counts, one per run."""
    ntiles = (T + 63) // 64
    best, bestn = None, 1
    for n in range(1, ntiles + 1):
        r = (ntiles + n - 1) // n
        if (ntiles + r - 1) // r != n:
            continue
        cost = ((nheads * n + ncu - 1) // ncu) * (r + 4)
        if best is None or cost < best:
            best, bestn = cost, n
    if bestn == 1:
        return [ntiles]
    r0 = min((ntiles + bestn - 1) // bestn, ntiles - (bestn - 1))
    rest = ntiles - r0
    rb, rx = divmod(rest, bestn - 1)
    return [r0] + [rb + (1 if k < rx else 0) for k in range(bestn - 1)]


def mfma_flops(B, H, T, ncu):
    """Matrix-core flops the run-streaming kernel executes per launch, from its
    instruction shape: every v_mfma_f32_16x16x32_bf16 is 2*16*16*32 = 16384
    flops.  Per 16-token chunk, each of the four matrix waves issues 6 for the
    readout (split state x split Qt), 1 for scores x V and 4 for the state
    update (split Kt^T x V): 11; one walker wave forms the chunk's causal
    scores (split Kt x split Qt) with 6.  A run with a predecessor corrects its
    two held tiles (8 chunks) with 6 more per chunk and matrix wave."""
    nheads = B * H
    ntiles = (T + 63) // 64
    runs = run_plan(nheads, T, ncu)
    chunks = nheads * ntiles * 4
    held_chunks = nheads * sum(4 * min(2, r) for r in runs[1:])
    instrs = chunks * (4 * 11 + 6) + held_chunks * 4 * 6
    return instrs * 16384, instrs


def algorithmic_flops(B, H, T, dk, dv):
    """Flops of the recurrent form per token: 5 dk dv for the mean update
    (decay, gated outer product) and readout, plus about 12 dk for the
    precision recursion and the gates."""
    return B * H * T * (5 * dk * dv + 12 * dk)


def kernel_source_hash():
    h = hashlib.sha256()
    for n in SOURCES:
        with open(os.path.join(ROOT, "bius_scan_sequence_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# Measured traffic of another workload's forward kernel (`--traffic-config`):
# the kernel's name, the summary file and the workload's algorithmic bytes.
TRAFFIC_CONFIGS = {
    "long_bf16": ("kla_fwd_kernel<128, 128, true", os.path.join(ROOT, "profiles", "kla_fwd_long_bf16_traffic.json"),
                  "long_bf16 (B2 H16 T16384 d128, bf16)", (2, 16, 16384, 128, 128, 2)),
}


def summarize_traffic(fetch_dir, write_dir, config=None):
    """Write the measured-traffic summary from two rocprofv3 counter runs of
    `bench.py --copy-mb 256` (one with FETCH_SIZE, one with WRITE_SIZE), or, for
    `config`, of `bench.py --configs <config> --copy-mb 256`.

    The counters are read per dispatch in KiB.  Each is scaled by what it reads
    for a kernel of known traffic in the same run: the float32 -> bfloat16 cast
    that converts one [8,8,2048,64] input (33554432 B read, 16777216 B written)."""
    import csv
    import glob

    def per_kernel(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        tot = {}
        for r in rows:
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
        fwd = [v for (k, _), v in tot.items() if kernel in k]
        ref = [v for (k, _), v in sorted(tot.items(), key=lambda kv: int(kv[0][1])) if "bfloat16_copy_kernel" in k]
        if config is not None:  # the run's last five casts: the reference (the inputs' own casts come first)
            ref = ref[-5:]
        if not fwd or not ref:
            raise SystemExit(f"no {counter} rows for the forward kernel or the reference cast in {d}")
        return sum(fwd) / len(fwd), len(fwd), sum(ref) / len(ref)

    if config is None:
        kernel, out_path, label, shape = KERNEL, TRAFFIC_FILE, "lm45m_bf16 (B8 H8 T2048 d64, bf16)", (8, 8, 2048, 64, 64, 2)
        runs = ("python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline --copy-mb 256", "")
    else:
        kernel, out_path, label, shape = TRAFFIC_CONFIGS[config]
        runs = (f"python3 bench.py --configs {config} --no-cpu-baseline --copy-mb 256", f" --traffic-config {config}")
    fetch, n, ref_fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write, _, ref_write = per_kernel(write_dir, "WRITE_SIZE")
    fetch_scale = 33554432 / 1024 / ref_fetch
    write_scale = 16777216 / 1024 / ref_write
    rd = fetch * 1024 * fetch_scale
    wr = write * 1024 * write_scale
    out = {
        "kernel": kernel, "workload": label,
        "fetch_size_kib_per_launch": fetch, "write_size_kib_per_launch": write, "launches": n,
        "reference_kernel": "torch float32->bfloat16 cast of one [8,8,2048,64] tensor "
                            "(33554432 B read, 16777216 B written per launch)",
        "reference_fetch_kib": ref_fetch, "reference_write_kib": ref_write,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": algorithmic_bytes(*shape),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o bench -- {runs[0]}",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o bench -- {runs[0]}",
            f"python3 bench.py --traffic-from <out>/fetch <out>/write{runs[1]}",
        ],
    }
    if config is None:  # the bench line uses it only while the kernel's sources are unchanged
        out["source_sha256"] = kernel_source_hash()
    out["traffic_ratio"] = out["hbm_bytes_per_launch"] / out["algorithmic_bytes_per_launch"]
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: out[k] for k in ("hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch",
                                          "fetch_scale", "write_scale", "launches")}))


def device_copy_bandwidth(dev, stream, mb=512, reps=5):
    """Bandwidth of a plain device-to-device copy of `mb` MB (read + write
    bytes over time, HIP events on the stream), larger than the 256 MB
    last-level cache: the second denominator for the roofline fraction."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / secs / 1e9


_ORACLE_X = None  # the workload's inputs, inherited by forked oracle workers


def _oracle_heads(rows):
    """Oracle over a contiguous block of (b, h) pairs (flattened head rows)."""
    from oracle import kla_forward_f64
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec", "lambda0", "M0")
    x = _ORACLE_X
    B, H = x["q"].shape[:2]
    sub = {n: x[n].reshape((B * H,) + x[n].shape[2:])[rows[0]:rows[1]][None] for n in names}
    y, _, _ = kla_forward_f64(*(sub[n] for n in names))
    return y[0]


def cpu_baseline(x):
    """The float64 oracle, as it stands, on the whole workload (all heads, all
    tokens) on the host, in this process before the GPU is touched: once on
    one core (the whole batch in one vectorised call), then split into n
    contiguous blocks of (b, h) pairs over a pool of n forked processes,
    n = the cores this process may run on (at most 16, the host share of one
    GPU on an eight-GPU node).  `value` is the n-core rate; the 1-core rate is reported beside
    it.  Returns the JSON object and the oracle's y for the parity margin."""
    import multiprocessing as mp
    import numpy as np
    from oracle import kla_forward_f64
    global _ORACLE_X
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec", "lambda0", "M0")
    B, H, T, _ = x["q"].shape
    t0 = time.perf_counter()
    y, _, _ = kla_forward_f64(*(x[n] for n in names))
    wall1 = time.perf_counter() - t0
    n = max(1, min(16, len(os.sched_getaffinity(0)), B * H))
    bounds = [(B * H * i // n, B * H * (i + 1) // n) for i in range(n)]
    _ORACLE_X = x
    ctx = mp.get_context("fork")
    with ctx.Pool(n) as pool:
        pool.map(_oracle_heads, [(0, 1)] * n)  # untimed: start the workers and import the oracle
        t0 = time.perf_counter()
        parts = pool.map(_oracle_heads, bounds)
        walln = time.perf_counter() - t0
    _ORACLE_X = None
    yn = np.concatenate(parts).reshape(y.shape)
    if not np.array_equal(yn, y):
        raise RuntimeError("the pooled oracle disagrees with the single-process oracle")
    tokens = B * H * T
    return {"value": tokens / walln, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "value_1core": tokens / wall1,
            "sample": f"whole {WORKLOAD} workload ({B * H} heads x {T} tokens): {walln:.2f} s wall on {n} "
                      f"processes ({B * H} heads in {n} blocks, results gathered); {wall1:.2f} s on one core "
                      f"(one vectorised call)"}, y


CONFIGS = ("lm45m_bf16", "lm180m_bf16", "long_bf16", "chains_f32", "decode_lm45m_bf16", "decode_b256_bf16",
           "bwd_lm45m_bf16", "bwd_long_bf16", "ou_lm45m_bf16", "pro_lm45m_bf16", "vprec_lm45m_bf16")


def vprec_algorithmic_bytes(B, H, T, dk, dv, esz):
    """Bytes of the variant with the value precision per value channel: per
    token q, k, log_decay, proc_noise (d_k each), v and val_prec (d_v each)
    read and y (d_v) written; per head the fp32 d_k x d_v precision and mean
    out (no state in)."""
    return B * H * T * ((4 * dk + 3 * dv) * esz) + B * H * dk * dv * 4 * 2


def ou_algorithmic_bytes(B, H, T, dk, dv, esz):
    """The forward's bytes with the OU prior in continuous time: per token q,
    k, dt, val_prec (d_k each) and v read, y written; per (h, i) theta and
    sigma2; per head the fp32 state in and out."""
    return B * H * T * ((4 * dk + dv) * esz + dv * esz) + H * dk * 8 + B * H * (dk + dk * dv) * 4 * 2


def prologue_algorithmic_bytes(B, H, T, dk, dv, esz, width=4):
    """Bytes of the forward pass on raw projections: per token the raw xq, xk,
    dt_raw, vp_raw (d_k each) and xv read, y written; per (h, channel) the
    convolution taps and biases of q, k, v and per (h, i) theta and sigma2;
    per head the fp32 state in and out.  (The three tokens of history each
    segment's convolution reads are counted once: they are the previous
    segment's.)"""
    return (B * H * T * ((4 * dk + dv) * esz + dv * esz) + H * (2 * dk + dv) * (width + 1) * 4 + H * dk * 8
            + B * H * (dk + dk * dv) * 4 * 2)


def backward_algorithmic_bytes(B, H, T, dk, dv, esz):
    """Bytes the backward pass must move: per token the six inputs and dL/dy
    read in the input dtype plus the float32 precision path, the six input
    gradients written in the input dtype; per head the float32 state in
    (lambda0, M0) read and its gradients written."""
    per_token = (5 * dk + dv) * esz + dv * esz + 4 * dk + (5 * dk + dv) * esz
    state = B * H * (dk + dk * dv) * 4 * 2
    return B * H * T * per_token + state


def run_configs(only, copies, copy_mb=0):
    """Kernel time of each workload at its full shape, one JSON line per
    workload: forward workloads as 5 warm-up and 20 timed calls over rotating
    device-side input copies, the precision-only scan as 1 warm-up and 3
    timed calls, with HIP events on the launch stream around every call;
    decode workloads as 10 warm-up and 100 timed back-to-back calls between
    one event pair, then the same 100 calls captured in a HIP graph and
    replayed five times."""
    import numpy as np
    import torch
    import bius_scan_sequence_amd as K
    import kla_inputs as KI
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    for name in CONFIGS:
        if only and name not in only:
            continue
        w = KI.workload(name)
        print(f"[config] {name}", file=sys.stderr, flush=True)
        if name == "chains_f32":
            B, H, T, D = 1, 1024, 65536, 64
            x = KI.make_precision_inputs_torch(B=B, H=H, T=T, D=D, device=dev)
            out = (torch.empty((B, H, T, D), dtype=torch.float32, device=dev),
                   torch.empty((B, H, D), dtype=torch.float32, device=dev))
            ws = K.Workspace(dev)
            calls, warm = 3, 1
            run = lambda i: K.precision_scan(x["log_decay"], x["proc_noise"], x["obs_prec"], x["lambda0"],
                                             workspace=ws, out=out)
            units, unit, abytes = B * H * T * D, "elements/s", 16 * B * H * T * D
        elif w.kind == "decode":
            # One token per head, the state updated in place; enough input and
            # state copies rotate that the set exceeds the 256 MB last-level cache.
            B, H, dk, dv = w.B, w.H, w.dk, w.dv
            abytes = algorithmic_bytes(B, H, 1, dk, dv, 2)
            ncopy = max(2, min(64, int(1.2e9 // abytes)))
            xs = []
            for c in range(ncopy):
                xc = KI.make_forward_inputs_torch(w, seed=w.seed + c, device=dev)
                xc = {n: (t.view(B, H, -1) if n in ("q", "k", "v", "log_decay", "proc_noise", "val_prec") else t)
                      for n, t in xc.items()}
                xs.append(xc)
            ys = [torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]
            ws = K.Workspace(dev)
            calls, warm = 100, 10

            def run(i):
                xc = xs[i % ncopy]
                return K.decode_step(xc["q"], xc["k"], xc["v"], xc["log_decay"], xc["proc_noise"], xc["val_prec"],
                                     xc["lambda0"], xc["M0"], out=(ys[i % ncopy], xc["lambda0"], xc["M0"]))
            units, unit = B * H, "head-steps/s"
            # A decode call lasts a few microseconds, less than an event pair
            # around each call adds; time back-to-back calls instead (what a
            # generation loop sees, launch gaps included).
            for i in range(warm):
                run(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(calls):
                run(i)
            e1.record(stream)
            torch.cuda.synchronize()
            mean_s = e0.elapsed_time(e1) / 1e3 / calls
            # The same `calls` steps captured once in a HIP graph and replayed,
            # as a serving loop would run them: no per-call host launch cost.
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    run(i)
            g.replay()
            torch.cuda.synchronize()
            reps = 5
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_s = e0.elapsed_time(e1) / 1e3 / (reps * calls)
            print(json.dumps({"config": name, "calls": calls, "timing": "back-to-back",
                              "kernel_ms_mean": mean_s * 1e3, "value": units / mean_s, "unit": unit,
                              "algorithmic_bytes": abytes, "achieved_GBps": abytes / mean_s / 1e9,
                              "frac_of_8TBps": abytes / mean_s / 8e12,
                              "graph": {"ms_per_step": graph_s * 1e3, "value": units / graph_s,
                                        "frac_of_8TBps": abytes / graph_s / 8e12}}), flush=True)
            g = None
            x = xs = ys = run = None
            torch.cuda.empty_cache()
            continue
        elif w.kind == "forward_ou":
            B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
            esz = 2 if w.dtype == "bf16" else 4
            abytes = ou_algorithmic_bytes(B, H, T, dk, dv, esz)
            ncopy = max(1, min(copies, int(1.2e9 // abytes)))
            xs = [KI.make_ou_inputs_torch(w, seed=w.seed + c, device=dev) for c in range(ncopy)]
            outs = [(torch.empty((B, H, T, dv), dtype=xs[0]["q"].dtype, device=dev),
                     torch.empty((B, H, dk), dtype=torch.float32, device=dev),
                     torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)) for _ in range(ncopy)]
            ws = K.Workspace(dev)
            calls, warm = 20, 5

            def run(i):
                xc = xs[i % ncopy]
                return K.forward_ou(xc["q"], xc["k"], xc["v"], xc["dt"], xc["theta"], xc["sigma2"], xc["val_prec"],
                                    xc["lambda0"], xc["M0"], workspace=ws, out=outs[i % ncopy])
            units, unit = B * H * T, "tokens/s"
        elif w.kind == "forward_prologue":
            B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
            esz = 2 if w.dtype == "bf16" else 4
            abytes = prologue_algorithmic_bytes(B, H, T, dk, dv, esz)
            ncopy = max(1, min(copies, int(1.2e9 // abytes)))
            xs = [KI.make_prologue_inputs_torch(w, seed=w.seed + c, device=dev) for c in range(ncopy)]
            outs = [(torch.empty((B, H, T, dv), dtype=xs[0]["xq"].dtype, device=dev),
                     torch.empty((B, H, dk), dtype=torch.float32, device=dev),
                     torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)) for _ in range(ncopy)]
            ws = K.Workspace(dev)
            calls, warm = 20, 5

            def run(i):
                xc = xs[i % ncopy]
                return K.forward_prologue(xc["xq"], xc["xk"], xc["xv"], xc["dt_raw"], xc["theta"], xc["sigma2"],
                                          xc["vp_raw"], xc["conv_w"], xc["conv_b"], xc["lambda0"], xc["M0"],
                                          workspace=ws, out=outs[i % ncopy])
            units, unit = B * H * T, "tokens/s"
        elif w.kind == "forward_vprec":
            B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
            esz = 2 if w.dtype == "bf16" else 4
            abytes = vprec_algorithmic_bytes(B, H, T, dk, dv, esz)
            ncopy = max(1, min(copies, int(1.2e9 // abytes)))
            xs = [KI.make_vprec_inputs_torch(w, seed=w.seed + c, device=dev) for c in range(ncopy)]
            outs = [(torch.empty((B, H, T, dv), dtype=xs[0]["q"].dtype, device=dev),
                     torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev),
                     torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)) for _ in range(ncopy)]
            ws = K.Workspace(dev)
            calls, warm = 20, 5

            def run(i):
                xc = xs[i % ncopy]
                return K.forward_vprec(*(xc[n] for n in NAMES), out=outs[i % ncopy])
            units, unit = B * H * T, "tokens/s"
        elif w.kind == "backward":
            # One kla_backward call over the whole batch (all six kernels), on
            # rotating input copies; each copy's precision path comes from one
            # forward call before timing.
            B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
            esz = 2 if w.dtype == "bf16" else 4
            abytes = backward_algorithmic_bytes(B, H, T, dk, dv, esz)
            ncopy = max(1, min(copies, int(1.2e9 // abytes)))
            xs = []
            for c in range(ncopy):
                xc = KI.make_forward_inputs_torch(w, seed=w.seed + c, device=dev)
                xc["grad_y"] = KI.make_backward_grads_torch(w, seed=w.seed + c, device=dev)
                xc["lpath"] = K.forward(*(xc[n] for n in NAMES), xc["lambda0"], xc["M0"],
                                        return_lambda_path=True)[3]
                xc["out"] = tuple(torch.empty_like(xc[n]) for n in NAMES) + (
                    torch.empty_like(xc["lambda0"]), torch.empty_like(xc["M0"]))
                xs.append(xc)
            ws = K.Workspace(dev)
            calls, warm = 20, 5

            def run(i):
                xc = xs[i % ncopy]
                return K.backward(*(xc[n] for n in NAMES), xc["grad_y"], xc["lpath"], xc["lambda0"], xc["M0"],
                                  workspace=ws, out=xc["out"])
            units, unit = B * H * T, "tokens/s"
        else:
            B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
            esz = 2 if w.dtype == "bf16" else 4
            ncopy = max(1, min(copies, int(1.2e9 // (algorithmic_bytes(B, H, T, dk, dv, esz)))))
            xs = [KI.make_forward_inputs_torch(w, seed=w.seed + c, device=dev) for c in range(ncopy)]
            outs = [(torch.empty((B, H, T, dv), dtype=xs[0]["q"].dtype, device=dev),
                     torch.empty((B, H, dk), dtype=torch.float32, device=dev),
                     torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)) for _ in range(ncopy)]
            ws = K.Workspace(dev)
            calls, warm = 20, 5

            def run(i):
                xc = xs[i % ncopy]
                return K.forward(xc["q"], xc["k"], xc["v"], xc["log_decay"], xc["proc_noise"], xc["val_prec"],
                                 xc["lambda0"], xc["M0"], workspace=ws, out=outs[i % ncopy])
            units, unit, abytes = B * H * T, "tokens/s", algorithmic_bytes(B, H, T, dk, dv, esz)
        for i in range(warm):
            run(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for i in range(calls):
            ev[i][0].record(stream)
            run(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        if ws.error():
            raise RuntimeError(f"device reported workspace error {ws.error()} on {name}")
        mean_s = float(ms.mean()) / 1e3
        print(json.dumps({"config": name, "calls": calls, "kernel_ms_mean": float(ms.mean()),
                          "kernel_ms_median": float(np.median(ms)), "kernel_ms_min": float(ms.min()),
                          "kernel_ms_max": float(ms.max()), "value": units / mean_s, "unit": unit,
                          "algorithmic_bytes": abytes, "achieved_GBps": abytes / mean_s / 1e9,
                          "frac_of_8TBps": abytes / mean_s / 8e12}), flush=True)
        x = xs = outs = out = run = None
        torch.cuda.empty_cache()
    if copy_mb:
        # The reference of known traffic for hardware-counter runs: five
        # float32 -> bfloat16 casts of one [8,8,2048,64] tensor.
        src = torch.ones((8, 8, 2048, 64), dtype=torch.float32, device=dev)
        for _ in range(5):
            src.to(torch.bfloat16)
        torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=3, help="rotating input/output copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, run five plain device copies of this many MiB (a reference of known "
                         "traffic for hardware counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the measured-traffic summary from two rocprofv3 counter runs and exit")
    ap.add_argument("--traffic-config", choices=sorted(TRAFFIC_CONFIGS),
                    help="with --traffic-from: the counter runs were of `--configs NAME --copy-mb 256`")
    ap.add_argument("--configs", nargs="*", metavar="NAME",
                    help=f"instead of the headline line, time every workload at its full shape (or the named "
                         f"ones of {', '.join(CONFIGS)}), one JSON line each")
    args = ap.parse_args()
    if args.traffic_from:
        summarize_traffic(*args.traffic_from, config=args.traffic_config)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.configs is not None:
        run_configs(set(args.configs), args.copies, args.copy_mb)
        return

    import numpy as np
    import kla_inputs as KI

    w = KI.workload(WORKLOAD)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    x = KI.make_forward_inputs(w)
    # The host baseline runs first, while no process has touched the GPU.
    cb, y_ref = (None, None) if args.no_cpu_baseline else cpu_baseline(x)

    import torch
    import bius_scan_sequence_amd as K
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    copies = []
    for c in range(args.copies):
        d = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in names}
        d["lambda0"] = torch.from_numpy(x["lambda0"]).to(dev)
        d["M0"] = torch.from_numpy(x["M0"]).to(dev)
        d["y"] = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
        d["lamT"] = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        d["MT"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        copies.append(d)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    need = K.kla_forward_workspace_bytes(B, H, T, dk, dv)
    ws = K.Workspace(dev).get(need, sh)
    args_c = [(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_decay"].data_ptr(),
               d["proc_noise"].data_ptr(), d["val_prec"].data_ptr(), d["lambda0"].data_ptr(),
               d["M0"].data_ptr(), d["y"].data_ptr(), d["lamT"].data_ptr(), d["MT"].data_ptr(), None,
               B, H, T, dk, dv, K.KLA_BF16, ws.data_ptr(), ws.numel(), sh) for d in copies]

    def step(i):
        rc = K.kla_forward(*args_c[i % len(args_c)])
        if rc:
            raise K.KlaError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_mean_s = float(np.mean(kern_ms)) / 1e3
    if ws_err := K.kla_workspace_error(ws.data_ptr()):
        raise RuntimeError(f"device reported workspace error {ws_err}")

    eager_ms_per_step = wall / args.steps * 1e3
    eager_kern_mean_ms = kern_mean_s * 1e3
    # The same K steps launched as one captured HIP graph (the kernels of the
    # eager loop, in the same order over the same rotating copies; no memset
    # or allocation sits in a step): the host's per-call launch cost is gone,
    # as in a serving or training loop that replays its graph.  `value` and
    # `ms_per_step` come from this run; the eager figure is reported beside it.
    # (Skipped in the hardware-counter runs, --copy-mb, which average the
    # counters over the eager dispatches only.)
    ms_per_step = eager_ms_per_step
    if not args.copy_mb:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream(dev).cuda_stream
            for i in range(args.steps):
                a = list(args_c[i % len(args_c)])
                a[-1] = cs
                if K.kla_forward(*a):
                    raise RuntimeError("kla_forward failed during graph capture")
        graph.replay()  # untimed: the graph's first launch
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        g0.record(stream)
        graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
        # The kernels of one stream run one after another: the event pair
        # around the replay over K is the kernel's average launch duration.
        kern_mean_s = g0.elapsed_time(g1) / 1e3 / args.steps
        if ws_err := K.kla_workspace_error(ws.data_ptr()):
            raise RuntimeError(f"device reported workspace error {ws_err}")
    tokens = B * H * T
    abytes = algorithmic_bytes(B, H, T, dk, dv, 2)
    achieved = abytes / kern_mean_s / 1e9
    traffic = measured_traffic()
    copy_gbs = device_copy_bandwidth(dev, stream)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    mflops, minstr = mfma_flops(B, H, T, ncu)
    aflops = algorithmic_flops(B, H, T, dk, dv)
    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "T": T, "d_k": dk, "d_v": dv,
                   "inputs": "bf16", "scan": "fp32", "copies": args.copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": KERNEL, "algorithmic_bytes": abytes,
                     "kernel_ms_mean": kern_mean_s * 1e3,
                     "kernel_ms_mean_eager_events": eager_kern_mean_ms,
                     "kernel_ms_min_eager_events": float(np.min(kern_ms)),
                     "kernel_ms_max_eager_events": float(np.max(kern_ms)),
                     "device_copy_GBps": copy_gbs, "frac_of_device_copy": achieved / copy_gbs,
                     "traffic_ratio": (traffic / abytes) if traffic else None,
                     "mfma_frac": mflops / kern_mean_s / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                     "mfma": {"peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                              "executed_flops": mflops, "instructions": minstr,
                              "achieved": mflops / kern_mean_s / 1e12,
                              "frac": mflops / kern_mean_s / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                              "algorithmic_flops": aflops,
                              "algorithmic_frac": aflops / kern_mean_s / 1e12 / PEAK_MFMA_BF16_TFLOPS}},
        "cpu_baseline": None,
        "launch": {"timed": "eager calls" if args.copy_mb else "one captured HIP graph of the K steps",
                   "eager_ms_per_step": eager_ms_per_step, "eager_value": tokens / (eager_ms_per_step / 1e3)},
    }
    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_reference"] = {"mib": args.copy_mb, "launches": 5, "bytes_read": n * 4, "bytes_written": n * 4}
    if cb is not None:
        y_gpu = copies[0]["y"].float().cpu().numpy()
        out["cpu_baseline"] = cb
        # max |y - r| / (1e-2 + 2e-2 |r|) against the oracle (<= 1 passes the bf16 bar)
        out["parity_y_margin"] = float(np.max(np.abs(y_gpu - y_ref) / (1e-2 + 2e-2 * np.abs(y_ref))))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
