"""Host checks of bench.py's contract (no GPU): more than one GPU is refused
with a message, and the per-stage roofline record divides the method's
algorithmic work by the measured times against the right peaks."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_stage_record_fractions():
    cfg = wl.WORKLOADS[4]
    m, n, N, bits = 49152, 12288, 262144, 4
    st = {"hessian": 40.0, "prepare": 30.0, "quantize": 70.0, "pack": 0.2}
    rec = bench.stage_record(cfg, m, n, N, 1, bits, st)
    # H: n(n+1)N flops against the fp16 matrix-core peak
    assert rec["hessian"]["frac_peak"] == pytest.approx(n * (n + 1) * N / 40e-3 / 2.5e15)
    # U: (2/3) n^3 against float64
    assert rec["prepare"]["frac_peak"] == pytest.approx(2 / 3 * n ** 3 / 30e-3 / 78.6e12)
    # deferred update: m n (n - 128) against the fp32 matrix cores
    assert rec["quantize"]["update_frac_f32_peak"] == pytest.approx(m * n * (n - 128) / 70e-3 / 157.3e12)
    # pack: codes read, words written, against HBM
    assert rec["pack"]["frac_hbm"] == pytest.approx((m * n * (1 + bits / 8) + 8 * n) / 0.2e-3 / 8e12)
    # fp32 inputs take the fp32 matrix-core peak for the Hessian
    rec1 = bench.stage_record(wl.WORKLOADS[1], 256, 256, 2048, 1, 4, st)
    assert rec1["hessian"]["frac_peak"] == pytest.approx(256 * 257 * 2048 / 40e-3 / 157.3e12)
