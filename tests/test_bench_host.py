"""Host-side pieces of bench.py's measurement chain (CPU, no GPU): the
roofline arithmetic, the per-kernel table, the algorithmic flop count, the
HBM-traffic record keyed on the library digest, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layer_flops_is_three_gemms():
    # forward, data gradient and filter gradient: 3 x 2*O*Kc*N each
    for w in wl.WORKLOADS.values():
        for layer in w.layers:
            sh = layer.shape
            assert bench.layer_flops(sh) == 3 * 2 * sh.outC * sh.Kc * sh.N
    # AlexNet conv3-5 at batch 64: 200.96 GFLOP per step
    step = sum(bench.layer_flops(l.shape) for l in wl.WORKLOADS["c4"].layers)
    assert abs(step / 1e9 - 200.96) < 0.01


def test_kernel_table_and_roofline():
    stats = [  # two launches of a GEMM class under two tags, one HBM-bound kernel
        {"name": "gemm_f32_128x128_kk:wgrad", "launches": 2, "ms": 0.4, "flops": 2 * 24e9, "bytes": 2 * 150e6},
        {"name": "gemm_f32_128x128_kk:other", "launches": 1, "ms": 0.2, "flops": 24e9, "bytes": 150e6},
        {"name": "im2col_f32:fwd", "launches": 3, "ms": 0.09, "flops": 0.0, "bytes": 3 * 150e6},
    ]
    by_kernel, kernels = bench.kernel_table(stats, 157.3)
    g = kernels["gemm_f32_128x128_kk"]
    assert g["launches"] == 3 and abs(g["avg_us"] - 200.0) < 1e-9
    assert abs(g["TFLOPs"] - 3 * 24e9 / 0.6e-3 / 1e12) < 1e-9       # 120 TFLOP/s
    assert abs(g["share"] - 0.6 / 0.69) < 1e-12
    # intensity 160 flop/B is above the fp32 ridge: attainable = peak
    assert g["attainable_TFLOPs"] == 157.3
    h = kernels["im2col_f32"]
    assert abs(h["GBps"] - 450e6 / 0.09e-3 / 1e9) < 1e-6 and "TFLOPs" not in h
    r = bench.roofline_of(by_kernel, "gemm_f32_128x128_kk", 157.3)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - 120.0) < 1e-9 and abs(r["frac"] - 120.0 / 157.3) < 1e-12
    assert abs(r["avg_launch_us"] - 200.0) < 1e-9 and r["launches"] == 3
    r = bench.roofline_of(by_kernel, "im2col_f32", 157.3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBPS


def test_attainable_below_the_ridge():
    # 1 flop per byte at 8 TB/s: 8 TFLOP/s attainable, whatever the MFMA peak
    assert abs(bench.attainable_tf(8e12, 8e12, 157.3) - 8.0) < 1e-9


def test_traffic_record_follows_the_library_digest(monkeypatch):
    d = bench.library_digest()
    assert len(d) == 64 and d == bench.library_digest()
    rec = bench.recorded_traffic("gemm_f32_128x128_kk")
    text = open(os.path.join(ROOT, "profiles", "traffic_alexnet_conv3-5_f32.txt")).read()
    if f"traffic_library_sha256: {d}" in text:
        assert rec is not None and rec[1] == os.path.join("profiles", "traffic_alexnet_conv3-5_f32.txt")
        assert f"traffic_bytes_per_launch: {int(rec[0])}" in text
    else:
        assert rec is None  # the library changed since the counters were taken
    assert bench.recorded_traffic("no_such_kernel") is None
    # any other library (a different digest) gets no recorded traffic
    monkeypatch.setattr(bench, "library_digest", lambda: "0" * 64)
    assert bench.recorded_traffic("gemm_f32_128x128_kk") is None


def test_forward_labels():
    assert bench.forward_label({"implicit": False, "fwd_form": "nhwc"}) == "explicit (im2col + GEMM)"
    assert bench.forward_label({"implicit": True, "fwd_form": "nhwc"}) == "implicit (NHWC)"
    assert bench.forward_label({"implicit": True, "fwd_form": "pointwise"}).startswith("pointwise")


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
