"""Per-phase timeline of the run-streaming forward (kla_fwd_run_kernel) and of
the backward chunk kernel (kla_bwd_chunk_kernel).

    python3 bius_scan_sequence_amd/build.py --timeline
    python3 bius_scan_sequence_amd/timeline.py [--config lm45m_bf16] [--calls 5]
    python3 bius_scan_sequence_amd/timeline.py --backward [--config bwd_lm45m_bf16]
    python3 bius_scan_sequence_amd/timeline.py --segmented [--config long_bf16]

The timeline build (libkla_timeline.so) compiles the run kernel with
-DKLA_TIMELINE: the first lane of wave 0 (a walker) and of wave 4 (a matrix
wave) of every workgroup records the 100 MHz real-time counter at fixed points.
This script runs the forward on a workload's synthetic inputs (device-side
generator, as the benchmark), reads the stamps of the last call and prints the
median duration of each phase over the workgroups.  The stamps themselves cost
a little time, so phases read slightly longer than in the ordinary build.

Slots (per workgroup): role 0 = walkers, role 1 = matrix waves.
  both roles   0 entry, 1 ticket read (run and tile range known)
  walkers      2 first tile staged; step j < 8 at 3 + 7 j + k:
               k = 0 step start, 1 composition walk and chunk scan, 2 gate walk,
               3 operands and bookkeeping stored, 4 walker/matrix sync passed,
               5 causal scores, 6 exact-path check and next tile staged
               62 run index, 63 tiles in the run (values, not times)
  matrix       2 window walk done (precision entering the run), 3 + 2 j after
               the work of tile j - 1, 4 + 2 j before the step's barrier;
               40 loop done, 41 look-back start, 42 look-back done,
               43 inclusive mean published, 44 end (held tiles corrected);
               path counters (values): 50 window tiles composed, 51 mid-run
               resolves of the entering mean, 52 chunks on the exact path
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
TL_LIB = os.path.join(PKG, "libkla_timeline.so")
SLOTS, GROUPS = 64, 4096
NAMES = ("q", "k", "v", "log_decay", "proc_noise", "val_prec")


def _us(d):
    return d / 100.0  # 100 MHz counter


def _med(a):
    a = np.asarray(a, np.float64)
    return float(np.median(a)) if a.size else float("nan")


def run(config: str = "lm45m_bf16", calls: int = 5, lib_path: str = TL_LIB) -> str:
    import torch
    sys.path.insert(0, os.path.dirname(PKG))
    import kla_inputs as KI

    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} missing: build it with bius_scan_sequence_amd/build.py --timeline")
    lib = ctypes.CDLL(lib_path)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.kla_forward_workspace_bytes.restype = sz
    lib.kla_forward_workspace_bytes.argtypes = [i] * 5
    lib.kla_forward.restype = i
    lib.kla_forward.argtypes = [vp] * 12 + [i] * 6 + [vp, sz, vp]
    lib.kla_workspace_init.argtypes = [vp, sz, vp]
    lib.kla_workspace_init.restype = i
    lib.kla_timeline_read.argtypes = [vp, sz]
    lib.kla_timeline_read.restype = i
    lib.kla_timeline_clear.restype = i

    w = KI.workload(config)
    if not (w.dk == 64 and w.dv == 64 and w.dtype == "bf16"):
        raise ValueError(f"{config}: the run kernel serves bf16 inputs at d_k = d_v = 64")
    dev = torch.device("cuda", 0)
    x = KI.make_forward_inputs_torch(w, device=dev)
    B, H, T = w.B, w.H, w.T
    y = torch.empty((B, H, T, 64), dtype=torch.bfloat16, device=dev)
    lT = torch.empty((B, H, 64), device=dev)
    MT = torch.empty((B, H, 64, 64), device=dev)
    need = lib.kla_forward_workspace_bytes(B, H, T, 64, 64)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.kla_workspace_init(ws.data_ptr(), need, st)
    if rc != 0:
        raise RuntimeError(f"kla_workspace_init: status {rc}")
    args = ([x[n].data_ptr() for n in NAMES] + [None, None, y.data_ptr(), lT.data_ptr(), MT.data_ptr(), None,
                                                B, H, T, 64, 64, 1, ws.data_ptr(), need, st])
    for _ in range(calls):
        assert lib.kla_forward(*args) == 0
    torch.cuda.synchronize()
    assert lib.kla_timeline_clear() == 0
    assert lib.kla_forward(*args) == 0
    torch.cuda.synchronize()
    buf = np.zeros(GROUPS * 2 * SLOTS, dtype=np.uint64)
    assert lib.kla_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    S = buf.reshape(GROUPS, 2, SLOTS).astype(np.int64)
    ngroups = int(np.count_nonzero(S[:, 0, 0]))
    S = S[:ngroups]
    W, X = S[:, 0], S[:, 1]
    runs, ntl = W[:, 62], W[:, 63]
    t0 = min(W[:, 0].min(), X[:, 0].min())

    out = []
    p = out.append
    p(f"kla_fwd_run_kernel timeline: {config} (B{B} H{H} T{T} d64 bf16), {ngroups} workgroups, "
      f"{int(runs.max()) + 1} runs per head, tiles per run {sorted(set(ntl.tolist()), reverse=True)}")
    p("medians over workgroups, in us (100 MHz real-time counter; the stamps add a little time)")
    p("")
    p("| phase | us |")
    p("|---|---|")
    p(f"| entry of the workgroups (spread: median / max after the first) | {_us(_med(W[:, 0] - t0)):.2f} / "
      f"{_us((W[:, 0] - t0).max()):.2f} |")
    p(f"| ticket and epoch read | {_us(_med(W[:, 1] - W[:, 0])):.2f} |")
    p(f"| first tile staged (walkers) | {_us(_med(W[:, 2] - W[:, 1])):.2f} |")
    sel = runs > 0
    if sel.any():
        p(f"| window walk, runs after the first (matrix waves, beside the walkers' first step) | "
          f"{_us(_med(X[sel, 2] - X[sel, 1])):.2f} |")
    # Walker steps: the middle steps of every run (not the first, not the last).
    names = ["composition walk + chunk scan", "gate walk", "operands and bookkeeping stored",
             "walker / matrix sync", "causal scores", "exact-path check, next tile staged"]
    per = {n: [] for n in names}
    waits, steps = [], []
    for j in range(1, 7):
        b = 3 + 7 * j
        ok = (ntl > j + 1) & (W[:, b] > 0) & (W[:, b + 7] > 0)
        if not ok.any():
            continue
        for k, n in enumerate(names):
            per[n].extend((W[ok, b + k + 1] - W[ok, b + k]).tolist())
        waits.extend((W[ok, b + 7] - W[ok, b + 6]).tolist())
        steps.extend((W[ok, b + 7] - W[ok, b]).tolist())
    for n in names:
        p(f"| walker step: {n} | {_us(_med(per[n])):.2f} |")
    p(f"| walker step: barrier (waiting for the matrix waves) | {_us(_med(waits)):.2f} |")
    p(f"| **walker step, total** | **{_us(_med(steps)):.2f}** |")
    mw = []
    for j in range(2, 8):
        ok = (ntl > j) & (X[:, 3 + 2 * j] > 0) & (X[:, 3 + 2 * (j - 1)] > 0)
        mw.extend((X[ok, 3 + 2 * j] - X[ok, 4 + 2 * (j - 1)]).tolist())
    p(f"| matrix step: four chunks of one tile (from the barrier to the end of its work) | {_us(_med(mw)):.2f} |")
    p(f"| loop done (from the first entry) | {_us(_med(X[:, 40] - t0)):.2f} |")
    held = X[:, 41] > 0
    if held.any():
        p(f"| end of loop to look-back start (aggregate published), runs after the first | "
          f"{_us(_med(X[held, 41] - X[held, 40])):.2f} |")
        p(f"| look-back (waiting for the earlier runs, folding their carries) | "
          f"{_us(_med(X[held, 42] - X[held, 41])):.2f} |")
        p(f"| inclusive mean published | {_us(_med(X[held, 43] - X[held, 42])):.2f} |")
        p(f"| held tiles corrected | {_us(_med(X[held, 44] - X[held, 43])):.2f} |")
    p("")
    p("| run | workgroups | loop done | end |")
    p("|---|---|---|---|")
    for r in range(int(runs.max()) + 1):
        m = runs == r
        p(f"| {r} | {int(m.sum())} | {_us(_med(X[m, 40] - t0)):.2f} | {_us(_med(X[m, 44] - t0)):.2f} |")
    p("")
    p(f"paths: window tiles composed per later run (median / max) {_med(X[sel, 50]):.0f} / {int(X[sel, 50].max()) if sel.any() else 0}; "
      f"mid-run resolves {int(X[:, 51].sum())}; chunks on the exact path {int(X[:, 52].sum())} "
      f"(matrix wave 4 of each workgroup)")
    p(f"kernel span (first entry to last end): {_us(max(X[:, 44].max(), W[:, 0].max()) - t0):.2f} us")
    return "\n".join(out)


BWD_PHASES = ("segment start: state loads issued", "work before the chunk loop",
              "barrier before the chunk loop", "mean tiles M_c^T", "outputs (dq, dg, e / dv)",
              "adjoint update", "operands of the next chunk", "barrier after the last chunk of a segment")


def run_backward(config: str = "bwd_lm45m_bf16", calls: int = 3, lib_path: str = TL_LIB) -> str:
    """Per-wave phase sums of kla_bwd_chunk_kernel (the timeline build's s_memtime
    accumulators), averaged over the workgroups of the recorded call's last
    chunk-kernel launch, in us at the measured shader clock."""
    import time

    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} missing: build it with bius_scan_sequence_amd/build.py --timeline")
    os.environ["BIUS_KLA_LIB"] = lib_path
    import torch
    sys.path.insert(0, os.path.dirname(PKG))
    import bius_scan_sequence_amd as K
    import kla_inputs as KI

    lib = K.lib
    lib.kla_bwd_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.kla_bwd_timeline_read.restype = ctypes.c_int
    w = KI.workload(config)
    dev = torch.device("cuda", 0)
    x = KI.make_forward_inputs_torch(w, device=dev)
    gy = KI.make_backward_grads_torch(w, device=dev)
    lpath = K.forward(*(x[n] for n in NAMES), x["lambda0"], x["M0"], return_lambda_path=True)[3]
    ws = K.Workspace(dev)

    def call():
        return K.backward(*(x[n] for n in NAMES), gy, lpath, x["lambda0"], x["M0"], workspace=ws)

    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    P, G = 16, 4096
    buf = np.zeros(G * 8 * P, dtype=np.uint64)
    assert lib.kla_bwd_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    S = buf.reshape(G, 8, P).astype(np.float64)
    used = S[:, 0, 8] > 0
    S = S[used]
    life = S[:, :, 9]
    # The shader clock: s_memtime counts it; 2.4 GHz is the nominal rate.
    ghz = 2.4
    out = []
    p = out.append
    p(f"kla_bwd_chunk_kernel phases: {config} (B{w.B} H{w.H} T{w.T} d_k {w.dk} d_v {w.dv} {w.dtype}), "
      f"{int(used.sum())} workgroups, {S[:, 0, 8].mean():.1f} segments each (last launch of the call)")
    p(f"per-wave sums averaged over workgroups, us at {ghz} GHz; the stamps add a little time "
      f"(whole call {wall * 1e3:.2f} ms wall)")
    p("")
    p("| phase | " + " | ".join(f"wave {v}" for v in range(8)) + " |")
    p("|---|" + "---|" * 8)
    rows = [(0, BWD_PHASES[0]), (10, "staging: gates, cumulative decays, LDS writes (two barriers)"),
            (11, "staging: wait for the state loads and earlier stores"),
            (12, "next segment's input loads issued (a share per chunk)")] + \
        [(k, BWD_PHASES[k]) for k in range(1, 3)] + [(15, "barrier after the chunk before (and a flag read)")] + \
        [(3, BWD_PHASES[3])] + \
        [(13, "outputs, key waves: Xs = dY M_c^T, Ys = V H^T"), (14, "outputs, key waves: in-chunk dq, dg parts"),
         (4, BWD_PHASES[4] + " (key waves: the stores)")] + \
        [(k, BWD_PHASES[k]) for k in range(5, len(BWD_PHASES))]
    for k, n in rows:
        p(f"| {n} | " + " | ".join(f"{S[:, v, k].mean() / ghz / 1e3:.2f}" for v in range(8)) + " |")
    p("| **life of the wave** | " + " | ".join(f"**{life[:, v].mean() / ghz / 1e3:.2f}**" for v in range(8)) + " |")
    return "\n".join(out)


SEG_PHASES = ("ticket read", "inputs staged", "chunk aggregates (precision maps)", "precision carry",
              "gate walk", "intra-chunk scores", "chunk loop (local states)", "mean carry (publish, look-back, fold)",
              "carried-state readout and store")


def run_segmented(config: str = "long_bf16", calls: int = 3, lib_path: str = TL_LIB) -> str:
    """Per-section durations of the segmented forward (kla_fwd_kernel), one
    workgroup per segment: medians over the workgroups of the recorded call,
    the spread of the mean carry, and how many segments its look-back folded."""
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} missing: build it with bius_scan_sequence_amd/build.py --timeline")
    os.environ["BIUS_KLA_LIB"] = lib_path
    import torch
    sys.path.insert(0, os.path.dirname(PKG))
    import bius_scan_sequence_amd as K
    import kla_inputs as KI

    lib = K.lib
    lib.kla_seg_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.kla_seg_timeline_read.restype = ctypes.c_int
    lib.kla_seg_timeline_clear.restype = ctypes.c_int
    w = KI.workload(config)
    dev = torch.device("cuda", 0)
    x = KI.make_forward_inputs_torch(w, device=dev)
    ws = K.Workspace(dev)

    def call():
        return K.forward(*(x[n] for n in NAMES), x["lambda0"], x["M0"], workspace=ws)

    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    assert lib.kla_seg_timeline_clear() == 0
    call()
    torch.cuda.synchronize()
    S_, G = 16, 16384
    buf = np.zeros(G * S_, dtype=np.uint64)
    assert lib.kla_seg_timeline_read(buf.ctypes.data, buf.nbytes) == 0
    S = buf.reshape(G, S_).astype(np.int64)
    S = S[S[:, 9] > 0]
    if len(S) == 0:
        raise SystemExit(f"{config}: kla_forward ran no segmented kernel (bf16 at d_k = d_v = 64 takes the "
                         f"run-streaming kernel; use the plain timeline)")
    t0 = S[:, 0].min()
    out = []
    p = out.append
    p(f"kla_fwd_kernel (segmented) timeline: {config} (B{w.B} H{w.H} T{w.T} d_k {w.dk} d_v {w.dv} {w.dtype}), "
      f"{len(S)} workgroups (one segment each)")
    p("medians over workgroups, in us (100 MHz real-time counter; the stamps add a little time)")
    p("")
    p("| section | median us | 90th percentile us |")
    p("|---|---|---|")
    for k, n in enumerate(SEG_PHASES):
        d = (S[:, k + 1] - S[:, k]) / 100.0
        p(f"| {n} | {np.median(d):.2f} | {np.percentile(d, 90):.2f} |")
    life = (S[:, 9] - S[:, 0]) / 100.0
    p(f"| **workgroup life** | **{np.median(life):.2f}** | {np.percentile(life, 90):.2f} |")
    folded = S[:, 11]
    p("")
    vals, cnt = np.unique(folded, return_counts=True)
    p("mean look-back: segments folded (1 = the predecessor's inclusive state only) -> workgroups: " +
      ", ".join(f"{int(v)}: {int(c)}" for v, c in zip(vals, cnt)))
    p(f"kernel span (first entry to last end): {(S[:, 9].max() - t0) / 100.0:.1f} us; "
      f"workgroup entries spread over {(S[:, 0].max() - t0) / 100.0:.1f} us")
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", default=None)
    ap.add_argument("--calls", type=int, default=5, help="calls before the recorded one")
    ap.add_argument("--lib", default=TL_LIB, help="another timeline build of the library")
    ap.add_argument("--backward", action="store_true", help="the backward chunk kernel's phases")
    ap.add_argument("--segmented", action="store_true", help="the segmented forward's sections")
    a = ap.parse_args()
    if a.segmented:
        print(run_segmented(a.config or "long_bf16", a.calls, a.lib), flush=True)
    elif a.backward:
        print(run_backward(a.config or "bwd_lm45m_bf16", a.calls, a.lib), flush=True)
    else:
        print(run(a.config or "lm45m_bf16", a.calls, a.lib), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
