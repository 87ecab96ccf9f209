"""Host-side logic of bench.py (no GPU): the flop model, the power-sample summary and the
single-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rankmixer_inputs import PRODUCTION, WORKLOADS  # noqa: E402


def test_gemm_flops_add_up_to_the_step():
    """The six GEMMs are the step's flops: forward 2N*D*2H + 2N*H*D, backward twice that
    (N = B*T tokens), 18 N D H in all; 3.87e12 at B=1024, T=64, D=1280, k=2."""
    d = WORKLOADS[PRODUCTION].dims
    f = bench.gemm_flops(d)
    assert sum(f.values()) == pytest.approx(bench.step_flops(d), rel=1e-12)
    assert bench.step_flops(d) == pytest.approx(3.865e12, rel=1e-3)
    # each backward product has the flops of its forward partner
    assert f["gemm_dhid"] == f["gemm_dwout"] == f["gemm_down"]
    assert f["gemm_dw1"] == f["gemm_dh1"] == f["gemm_up"]


def test_power_summary_uses_the_timed_window_only(tmp_path):
    p = tmp_path / "power.csv"
    rows = ["# power_cap_uw 1400000000"]
    rows += [f"{100.0 + 0.02 * i:.3f},{1000 + i},{1500 + i}" for i in range(50)]   # t = 100.00 .. 100.98
    rows += ["101.500,N/A,N/A"]                                                      # a sample without data
    p.write_text("\n".join(rows) + "\n")
    s = bench.power_summary(str(p), 100.2, 100.4)                                    # samples 10 .. 20
    assert s["samples"] == 11
    assert s["avg_w"] == pytest.approx(1015.0)
    assert s["max_w"] == 1020.0
    assert s["gfx_mhz_avg"] == pytest.approx(1515.0)
    assert s["cap_w"] == pytest.approx(1400.0)
    assert "error" in bench.power_summary(str(p), 200.0, 201.0)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
