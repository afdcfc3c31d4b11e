"""bench.py's host-side contract, on the CPU: the one-GPU guard and the
roofline arithmetic of the JSON line (no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "8"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_roofline_entry_mfma_bound():
    # the skewed prefill gate/up launch: 2 * 131072 rows * 7168 * 4096 FLOPs
    flops = 2.0 * 131072 * 7168 * 4096
    e = bench.roofline_entry(flops, 13.2e9, 6.5, bench.PEAK_BF16_TFLOPS)
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s" and e["peak"] == bench.PEAK_BF16_TFLOPS
    assert e["achieved"] == pytest.approx(flops / 6.5e-3 / 1e12)
    assert e["frac"] == pytest.approx(e["achieved"] / bench.PEAK_BF16_TFLOPS)
    assert 0.46 < e["frac"] < 0.48


def test_roofline_entry_hbm_bound_below_the_ridge():
    # decode: 64 tokens, a few FLOPs per streamed weight byte
    nbytes, flops = 12.0e9, 30.0e9
    e = bench.roofline_entry(flops, nbytes, 1.92, bench.PEAK_BF16_TFLOPS)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == bench.PEAK_HBM_GBS
    assert e["achieved"] == pytest.approx(nbytes / 1.92e-3 / 1e9)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0)


def test_ridge_point_decides_the_bound():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)  # FLOP per byte
    assert bench.roofline_entry(0.99 * ridge * 1e9, 1e9, 1.0, bench.PEAK_BF16_TFLOPS)["bound"] == "hbm"
    assert bench.roofline_entry(1.01 * ridge * 1e9, 1e9, 1.0, bench.PEAK_BF16_TFLOPS)["bound"] == "mfma"
    ridge8 = bench.PEAK_FP8_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert ridge8 == pytest.approx(2 * ridge, rel=1e-3)
