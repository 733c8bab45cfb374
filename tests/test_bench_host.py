"""Host-side logic of bench.py, no GPU: the run plan it mirrors from the
library, the byte and flop counts behind the roofline fields, the traffic
summary from counter CSVs, and the one-GPU guard."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_lm45m():
    # per token (5 d_k + 2 d_v) bf16 elements, per head the fp32 state in and out
    assert bench.algorithmic_bytes(8, 8, 2048, 64, 64, 2) == 64 * 2048 * 896 + 64 * (64 + 4096) * 8
    assert bench.algorithmic_bytes(8, 8, 2048, 64, 64, 2) == 119_570_432


@pytest.mark.parametrize("nheads,T,ncu,expect", [
    (64, 2048, 256, [8, 8, 8, 8]),   # lm45m: one round of four 8-tile runs
    (192, 2048, 256, [32]),          # lm180m: one 32-tile run per head
    (1, 64, 256, [1]),
    (1, 100, 256, [1, 1]),           # two tiles, the second ragged
])
def test_run_plan(nheads, T, ncu, expect):
    runs = bench.run_plan(nheads, T, ncu)
    assert runs == expect
    assert sum(runs) == (T + 63) // 64


@pytest.mark.parametrize("nheads,T", [(64, 2048), (192, 2048), (7, 1000), (300, 64 * 37)])
def test_run_plan_is_cheapest(nheads, T):
    """Brute force over every run count: the plan's cost (rounds x (longest
    run + 4)) is the minimum, and its runs differ by at most one tile."""
    ntiles = (T + 63) // 64
    runs = bench.run_plan(nheads, T, 256)
    cost = lambda n, r: ((nheads * n + 255) // 256) * (r + 4)
    best = min(cost(n, (ntiles + n - 1) // n) for n in range(1, ntiles + 1)
               if (ntiles + (ntiles + n - 1) // n - 1) // ((ntiles + n - 1) // n) == n)
    assert cost(len(runs), max(runs)) == best
    assert max(runs) - min(runs) <= 1 or len(runs) == 1


def test_mfma_flops_lm45m():
    # 2048 tiles x 4 chunks x 50 instructions, plus the held tiles of runs 1..3
    flops, instrs = bench.mfma_flops(8, 8, 2048, 256)
    assert instrs == 64 * 32 * 4 * 50 + 64 * 3 * 8 * 4 * 6
    assert flops == instrs * 16384


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": d + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_config(tmp_path, monkeypatch):
    """The long_bf16 summary scales by the run's last five reference casts,
    not by the larger input casts before them."""
    cast = "void at::native::bfloat16_copy_kernel_cuda(...)"
    fwd = "void kla::kla_fwd_kernel<128, 128, true, 0>(kla::FwdParams)"
    big = [(cast, 4 * 16384.0)] * 6                 # the workload's own input casts
    ref_f, ref_w = [(cast, 16384.0)] * 5, [(cast, 16384.0)] * 5
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", big + [(fwd, 1000.0), (fwd, 1000.0)] + ref_f)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", big + [(fwd, 500.0), (fwd, 500.0)] + ref_w)
    out = tmp_path / "t.json"
    k, _, label, shape = bench.TRAFFIC_CONFIGS["long_bf16"]
    monkeypatch.setitem(bench.TRAFFIC_CONFIGS, "long_bf16", (k, str(out), label, shape))
    bench.summarize_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), config="long_bf16")
    t = json.loads(out.read_text())
    # reference: 33554432 B read and 16777216 B written per cast
    assert t["fetch_scale"] == pytest.approx(33554432 / 1024 / 16384.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["hbm_read_bytes_per_launch"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert t["hbm_write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert t["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(2, 16, 16384, 128, 128, 2)
    assert t["traffic_ratio"] == pytest.approx(t["hbm_bytes_per_launch"] / t["algorithmic_bytes_per_launch"])
    assert "source_sha256" not in t  # only the bench line's own summary is tied to its sources


def test_traffic_summary_missing_kernel(tmp_path):
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", [("void other(...)", 1.0)])
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", [("void other(...)", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), config="long_bf16")


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
