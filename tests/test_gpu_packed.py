"""GPU parity of the data gradient from a pre-packed filter.

d4r_conv_pack_filter writes the data gradient's operand Wmat^T once (a bit
copy: checked bit for bit against the transposed filter);
d4r_conv_backward_data_packed must then give the oracle's dx on every data
path the library has: dy read in place (f32, small Kc), dy copied (large Kc,
16-bit), the direct 1x1 path, and a strided kernel.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

# (batch, C, H, W, O, kH, kW, stride, padding)
CASES = [((3, 5, 11, 9, 37, 3, 3, 1, 1), "f32"),     # in place (Kc = 45)
         ((2, 40, 9, 9, 48, 5, 5, 1, 2), "f32"),     # copied (Kc = 1000 < 1024: in place) ...
         ((2, 130, 7, 7, 40, 3, 3, 1, 1), "f32"),    # ... and Kc = 1170: copied
         ((2, 130, 7, 7, 40, 3, 3, 1, 1), "bf16"),
         ((2, 24, 10, 12, 40, 3, 3, 2, 1), "f16"),   # stride 2
         ((3, 64, 8, 8, 40, 1, 1, 1, 0), "f32"),     # direct 1x1 path
         ((3, 64, 8, 8, 40, 1, 1, 1, 0), "f16"),
         ((1, 3, 35, 35, 16, 11, 11, 4, 2), "f32")]  # AlexNet conv1 geometry


@pytest.mark.parametrize("t,dt", CASES, ids=[f"{c}-{d}" for c, d in CASES])
def test_backward_data_packed_matches_oracle(t, dt):
    B, C, H, W, O, kH, kW, s, p = t
    sh = wl.ConvShape(B, C, H, W, kH, kW, s, p, O)
    ops = wl.random_conv(sh, dt, seed=sum(t) + 11)
    pl = d4r.ConvPlan(B, C, H, W, kH, kW, s, p, O, DT_CODE[dt])
    w, g = dev(ops["w"]), dev(ops["g"])
    wp = pl.pack_filter(w)
    dx = pl.backward_data_packed(wp, g)
    dx_plain = pl.backward_data(w, g)
    torch.cuda.synchronize()
    # the packed filter is a bit copy of Wmat^T
    assert torch.equal(wp, w.reshape(O, C * kH * kW).t().contiguous())
    ref = oracle.conv_backward_data(ops["g"].exact, ops["w"].exact, sh.x_shape(), s, p)
    assert rel_err(host(dx), ref) < TOL[dt]
    assert rel_err(host(dx), host(dx_plain)) < TOL[dt]


def test_packed_filter_reused_across_micro_batches():
    # one pack, several data gradients (gradient accumulation): each equals
    # the unpacked call on its own micro-batch
    w_ = wl.WORKLOADS["c4"]
    sh = w_.layers[2].shape.with_batch(2)
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, 3, 3, 1, 1, sh.outC, d4r.D4R_BF16)
    ops = wl.conv_inputs(w_, 2, "bf16", batch=2)
    w = dev(ops["w"])
    wp = pl.pack_filter(w)
    for k in range(3):
        g = dev(ops["g"]) * (1.0 + k)
        dx_p = pl.backward_data_packed(wp, g)
        dx = pl.backward_data(w, g)
        torch.cuda.synchronize()
        assert rel_err(host(dx_p), host(dx)) < TOL["bf16"], k
