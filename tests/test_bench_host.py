"""Host-side logic of bench.py (no GPU): the algorithmic work per launch
behind the roofline figures, the choice of bound, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_work_of_the_long_workload():
    wl = synth.WORKLOADS["long"]
    T = 1 * 8 * 65536
    # causal scan: Q, K, V read and O written in bf16; projections of Q and K,
    # phi(Q) S and the state update, 2 m d flops each per token
    assert bench.algorithmic("k_causal", "causal", wl) == {"bytes": 4 * 64 * 2 * T, "flops": 8 * 256 * 64 * T}
    # non-causal halves: K, V in (reduction) or Q in, O out (apply)
    for k in ("k_reduce", "k_apply"):
        assert bench.algorithmic(k, "noncausal", wl) == {"bytes": 2 * 64 * 2 * T, "flops": 4 * 256 * 64 * T}
    assert bench.algorithmic("k_span_scan", "causal", wl) == {"bytes": 0, "flops": 0}


def test_roofline_bound_follows_the_ridge_point():
    # bf16 causal: 256 flops per byte, below the ridge 2500/8 = 312.5 -> HBM-bound
    e = bench.roofline_entry("k_causal", "causal", synth.WORKLOADS["long"], 0.1, None)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s"
    assert e["achieved"] == pytest.approx(4 * 64 * 2 * 524288 / 1e-4 / 1e9, rel=1e-3)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0, rel=1e-3)
    # float32 wide causal scan on split 16-bit products: three products per
    # float32 product, 768 executed flops per byte against the bf16 ridge
    # 312.5 -> MFMA-bound at the bf16 peak, with the float32-equivalent rate
    wl = synth.WORKLOADS["wide"]
    flops = bench.algorithmic("k_causal", "causal", wl)["flops"]
    e = bench.roofline_entry("k_causal", "causal", wl, 30.0, None)
    assert e["bound"] == "mfma" and e["peak"] == 2500.0 and e["unit"] == "TFLOP/s"
    assert e["executed_flops_per_launch"] == 3 * flops
    assert e["achieved"] == pytest.approx(3 * flops / 30e-3 / 1e12, rel=1e-2)
    assert e["f32_equivalent_frac"] == pytest.approx(flops / 30e-3 / 1e12 / 157.3, rel=1e-2)


def test_roofline_of_float32_products(monkeypatch):
    # FAVOR_F32_MFMA=1: float32 products, 256 flops per byte against the
    # float32 ridge 157.3/8 -> MFMA-bound at the float32 peak
    monkeypatch.setenv("FAVOR_F32_MFMA", "1")
    e = bench.roofline_entry("k_causal", "causal", synth.WORKLOADS["wide"], 30.0, None)
    assert e["bound"] == "mfma" and e["peak"] == 157.3 and "arithmetic" not in e


def test_source_hash_covers_the_forward_kernels():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    for name in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "random_feature_approx_amd", "csrc", name))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
