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
