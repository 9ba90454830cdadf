"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the algorithmic byte counts behind the roofline,
the source-hash gate on the recorded counter traffic, and the counter summary's copy calibration."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", ["lmhead_b1_g4", "lmhead_b8_g7", "greedy_b64_g4"])
def test_algorithmic_bytes(name):
    w = synth.WORKLOADS[name]
    N = w.B * (w.gamma + 1)
    W, X, Y = w.V * w.d * 2, N * w.d * 2, N * w.V * 4
    gemm, step = bench.algorithmic_bytes(w, fused=True, with_logits=True)
    assert gemm == W + X + Y  # one pass over bf16 W and X, fp32 logits written once
    sampling = 0 if w.temperature == 0.0 else w.B * w.gamma * w.V * 4 + w.B * w.V * 8
    assert step == W + X + Y + sampling  # draft logits read once, the (target, draft) row pair at k read again
    _, unfused = bench.algorithmic_bytes(w, fused=False, with_logits=True)
    assert unfused == step + Y  # without the fused statistics the logits are read once more
    _, no_logits = bench.algorithmic_bytes(w, fused=True, with_logits=False)
    assert no_logits == step - Y


def test_recorded_traffic_follows_the_kernel_sources(monkeypatch):
    for (workload, layout), rec in bench.MEASURED_TRAFFIC.items():
        assert bench.measured_traffic(workload, layout) == rec["fetch_bytes"] + rec["write_bytes"]
        # A record whose sources have changed since the counters were taken no longer describes the kernel.
        stale = dict(rec, source_sha256="0" * 64)
        monkeypatch.setitem(bench.MEASURED_TRAFFIC, (workload, layout), stale)
        assert bench.measured_traffic(workload, layout) is None
    assert bench.measured_traffic("no_such_workload", "packed") is None


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, grid, value in rows:
            wr.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy(tmp_path, capsys):
    copy = "__amd_rocclr_copyBuffer"
    k = "void specdec::gemm::(anonymous namespace)::panel_kernel<4, 4, 8, 2, false, 0>(unsigned short const*)"
    # FETCH_SIZE reads half of the 256 MiB the copy moves (factor 2); WRITE_SIZE reads it whole (factor 1).
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 512, 131072.0), (k, 131072, 1000.0), (k, 131072, 1002.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 512, 262144.0), (k, 131072, 30.0), (k, 131072, 34.0)])
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    out = capsys.readouterr().out
    assert "FETCH_SIZE x2.0000, WRITE_SIZE x1.0000" in out
    # per dispatch: fetch 1001 KiB x 2, write 32 KiB x 1
    assert f"fetch_bytes={1001 * 2 * 1024} write_bytes={32 * 1024}" in out
    assert "| gemm::panel_kernel<4, 4, 8, 2, false, 0> | 131072 | 2 |" in out
