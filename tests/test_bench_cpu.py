"""bench.py's arithmetic and contract on the CPU: the step's host-link
bounds from the bytes each phase moves, the recorded counter traffic of the
dominant kernel, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from host_memory_streamed_amd import mt  # noqa: E402


def test_link_roofline_phase_and_duplex():
    w = mt.WORKLOADS["14b"]
    d, L = w.d_model, w.n_layers
    qkv = (w.n_heads + 2 * w.n_kv_heads) * w.head_dim
    layer_img = 2 * d * 4 + (qkv * d + d * w.n_heads * w.head_dim + 3 * d * w.ffn_dim) * 2
    fwd = 28.0e9
    stats = {"h2d_bytes": fwd + (L - 1) * layer_img, "d2h_bytes": 56.0e9}
    bw = {"h2d": 50e9, "d2h": 40e9}
    r = bench.link_roofline(w, stats, 2.0, bw, 2)
    assert r["fwd_h2d_bytes"] == pytest.approx(fwd)
    assert r["bwd_h2d_bytes"] == (L - 1) * layer_img
    # forward phase: loads only; backward phase: the slower direction
    t_phase = fwd / 50e9 + max((L - 1) * layer_img / 50e9, 56e9 / 40e9)
    assert r["t_link_phase_s"] == pytest.approx(t_phase, abs=1e-4)
    assert r["t_link_duplex_s"] == pytest.approx(max(stats["h2d_bytes"] / 50e9, 56e9 / 40e9), abs=1e-4)
    assert r["frac_phase"] == pytest.approx(t_phase / 2.0, abs=1e-4)
    assert r["tokens_s_phase"] == pytest.approx(w.batch * w.seq / t_phase, rel=1e-3)


def test_recorded_traffic_only_for_its_kernel_and_source():
    t = bench.recorded_traffic("gemm_nt_bf16")
    assert t is None or t > 0
    assert bench.recorded_traffic("gemm_tn_bf16") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_summary_weights_clean_dispatches_by_the_step_mix(tmp_path, capsys):
    """A synthetic kernel trace of two steps, each with four fast dispatches
    (grid 1000, 100 us) and one slow one (grid 9000, 500 us). In the kept
    step a copy kernel overlaps three of the fast ones, which also run
    slower (300 us) as a traced copy makes them wait. The clean subset then
    holds one fast and one slow dispatch (plain mean 300 us); weighting each
    grid size's clean mean by its share of the kept dispatches gives
    4/5 * 100 + 1/5 * 500 = 180 us, the step's own mix."""
    rows, t = [], 0
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]

    def add(name, dur_us, grid, start=None):
        nonlocal t
        t0 = t if start is None else start
        rows.append({"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t0 + dur_us * 1000,
                     "Grid_Size_X": grid})
        if start is None:
            t = t0 + dur_us * 1000 + 1000
    for step in range(2):
        base = t
        for i in range(4):
            slow = step == 1 and i < 3
            add("gemm_big_kernelIDF16bLi0EE_x", 300 if slow else 100, 1000)
        add("gemm_big_kernelIDF16bLi0EE_x", 500, 9000)
        if step == 1:   # one copy spanning the first three fast dispatches of the kept step
            add("__amd_rocclr_copyBuffer", (rows[-2]["Start_Timestamp"] - base) // 1000, 256, start=base)
    path = tmp_path / "kernel_trace.csv"
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)
    bench.summarize_kernel_trace(str(path), steps=2, skip=1, kernel_substr="gemm_big_kernelIDF16bLi0EE",
                                 flops_per_launch=1.8e8)
    out = capsys.readouterr().out
    assert "| the same, overlapping no copy kernel | 2 | 300.0 |" in out
    assert "| clean mean per grid size, weighted by the step's mix | 5 | 180.0 |" in out
    # 1.8e8 FLOP in 180 us
    assert "shape-weighted, no copy overlap: 1.0 TFLOP/s" in out
