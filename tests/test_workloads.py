"""Seeded input generator: determinism, shapes and dtype rounding."""
import numpy as np
import pytest

import workloads as wl


def test_config_shapes():
    c = wl.WORKLOADS
    a1 = c["c3"].layers[0].shape
    assert (a1.outH, a1.outW, a1.Kc, a1.N) == (55, 55, 363, 32 * 55 * 55)
    s2 = c["c5"].layers[2].shape
    assert (s2.outH, s2.outW) == (23, 40)
    assert c["c1"].layers[0].shape.y_shape() == (8, 6, 24, 24)
    assert c["c2"].layers[0].shape.y_shape() == (64, 16, 8, 8)
    assert [l.shape.outC for l in c["c4"].layers] == [384, 384, 256]
    # C4 stack flops per dtype (3 GEMMs x 3 layers)
    tot = sum(3 * l.shape.gemm_flops() for l in c["c4"].layers)
    assert abs(tot / 1e9 - 200.96) < 0.01


def test_seeded_determinism_and_prefix():
    w = wl.WORKLOADS["c2"]
    a = wl.conv_inputs(w, 0, "f32")
    b = wl.conv_inputs(w, 0, "f32")
    for k in a:
        assert np.array_equal(a[k].stored, b[k].stored)
    s = wl.conv_inputs(w, 0, "f32", batch=5)
    assert np.array_equal(s["x"].stored, a["x"].stored[:5])
    assert np.array_equal(s["g"].stored, a["g"].stored[:5])
    assert np.array_equal(s["w"].stored, a["w"].stored)


def test_distributions():
    w = wl.WORKLOADS["c4"]
    x = wl.conv_inputs(w, 1, "f32")["x"].exact
    assert x.min() == 0.0 and (x == 0).mean() > 0.4
    std = wl.conv_inputs(w, 1, "f32")["w"].exact.std()
    assert abs(std - np.sqrt(2 / 3456)) / np.sqrt(2 / 3456) < 0.02


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9,
                     3.0e38], dtype=np.float32)
    bits = wl.f32_to_bf16_bits(vals)
    assert [hex(b) for b in bits[:5]] == ["0x3f80", "0x3f80", "0x3f82", "0xc020", "0x3f80"]
    back = wl.bf16_bits_to_f64(bits)
    assert back[2] == 1.0 + 4 * 2.0 ** -8


def test_f16_and_exact_widening():
    op = wl.quantize(np.array([0.1, -3.0, 65504.0]), "f16")
    assert op.stored.dtype == np.uint16
    assert np.array_equal(op.exact, np.array([0.1, -3.0, 65504.0]).astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("key", list(wl.WORKLOADS))
def test_gemm_case_storage(key):
    w = wl.WORKLOADS[key]
    for i, c in enumerate(w.gemms):
        ops = wl.gemm_inputs(w, i, "f32")
        assert ops["A"].stored.size == c.M * c.K
        assert ops["B"].stored.size == c.K * c.N
        if c.flags & 1:
            assert ops["A"].stored.shape == (c.K, c.M)
        if c.flags & 2:
            assert ops["B"].stored.shape == (c.N, c.K)

