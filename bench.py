#!/usr/bin/env python3
"""Throughput of the KLA forward scan on one MI355X.

Workload lm45m_bf16: B=8, H=8, T=2048, d_k=d_v=64, bf16 inputs, fp32 scan,
seeded synthetic inputs (kla_inputs recipe).  One step = one kla_forward call
over the whole batch (precision scan, gates, chunked mean recursion, readout).
Inputs are resident in HBM before timing; three input/output copies rotate so
the 256 MB last-level cache cannot hold the working set between steps.

Prints one JSON line:
  value      tokens/s (B*H*T per step / wall time per step)
  roofline   dominant kernel (kla_fwd_kernel<64,64,bf16>): algorithmic bytes
             per launch / mean launch duration (HIP events on the launch
             stream), against the 8 TB/s HBM peak; traffic = measured HBM
             bytes per launch from committed counter profiles when they were
             taken on the current kernel sources, else null
  cpu_baseline  the float64 oracle on the host, timed on the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KLA fwd tokens/s (B*H*T) at dk=dv=64,T=2048; % of HBM roofline"
WORKLOAD = "lm45m_bf16"
PEAK_HBM_GBS = 8000.0
KERNEL = "kla_fwd_kernel<64, 64, true>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kla_fwd_lm45m_bf16_traffic.json")
SOURCES = ["kla_forward.hip", "kla_device.h", "kla_internal.h"]


def algorithmic_bytes(B, H, T, dk, dv, esz):
    """Bytes the method must move: per token q, k, log_decay, proc_noise,
    val_prec (d_k each) and v (d_v) read, y (d_v) written; per head the fp32
    state in (lambda0, M0) and out (lambda_T, M_T)."""
    per_token = (5 * dk + dv) * esz + dv * esz
    state = B * H * (dk + dk * dv) * 4 * 2
    return B * H * T * per_token + state


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


def cpu_baseline(x, y_gpu):
    """The float64 oracle, as it stands, on the whole workload (all 64 heads,
    2048 tokens) on the host; returns the JSON object and the parity margin."""
    import numpy as np
    from oracle import kla_forward_f64
    names = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    y, lT, MT = kla_forward_f64(*(x[n] for n in names), x["lambda0"], x["M0"])
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    B, H, T, _ = x["q"].shape
    cores = max(1, round(cpu / wall))
    margin = float(np.max(np.abs(y_gpu - y) / (1e-2 + 2e-2 * np.abs(y))))
    return {"value": B * H * T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"whole {WORKLOAD} workload ({B * H} heads x {T} tokens), one pass, "
                      f"{wall:.2f} s wall, {cpu:.2f} s CPU"}, margin


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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bius_scan_sequence_amd as K
    import kla_inputs as KI

    w = KI.workload(WORKLOAD)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    x = KI.make_forward_inputs(w)
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

    ms_per_step = wall / args.steps * 1e3
    tokens = B * H * T
    abytes = algorithmic_bytes(B, H, T, dk, dv, 2)
    achieved = abytes / kern_mean_s / 1e9
    traffic = measured_traffic()
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
                     "kernel_ms_min": float(np.min(kern_ms)), "kernel_ms_max": float(np.max(kern_ms))},
        "cpu_baseline": None,
    }
    if args.copy_mb:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_reference"] = {"mib": args.copy_mb, "launches": 5, "bytes_read": n * 4, "bytes_written": n * 4}
    if not args.no_cpu_baseline:
        y_gpu = copies[0]["y"].float().cpu().numpy()
        cb, margin = cpu_baseline(x, y_gpu)
        out["cpu_baseline"] = cb
        out["parity_y_margin"] = margin  # max |y-r| / (1e-2 + 2e-2|r|) vs the oracle
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
