"""GPU parity of the fused epilogues: conv + bias + ReLU and linear + bias
(+ ReLU) in one GEMM.

d4r_conv_forward_ex and d4r_gemm_bias_act apply the bias and ReLU in the
GEMM's store (or in the split-K reduction), so each result must equal the
unfused sequence (forward or d4r_gemm, then the bias and ReLU kernels) bit
for bit, and the oracle's relu(conv + bias) / relu(op(A) op(B) + bias) within
the dtype's tolerance.  Shapes cover ragged tiles, the 1x1 direct path, the
implicit GEMM and split K (checked through the profile recorder's launch
names); every dtype.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

# (batch, C, H, W, kH, kW, stride, pad, O); the planner splits K for every
# f32 case and for the 16-bit (1, 256, 6, 6) case, so both epilogue sites
# (GEMM store and split-K reduction) run in every dtype
CONV = [(2, 16, 9, 11, 3, 3, 1, 1, 40),
        (3, 8, 13, 13, 5, 5, 2, 2, 130),
        (2, 16, 5, 7, 1, 1, 1, 0, 24),
        (1, 256, 6, 6, 3, 3, 1, 1, 16)]


def _launch_names(fn):
    d4r.d4r_profile_reset()
    d4r.d4r_profile_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
        return [r["name"] for r in d4r.d4r_profile_read()]
    finally:
        d4r.d4r_profile_enable(False)
        d4r.d4r_profile_reset()


@pytest.mark.parametrize("t", CONV, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("implicit", [False, True])
def test_conv_forward_relu(t, dt, implicit):
    sh = wl.ConvShape(*t)
    ops = wl.random_conv(sh, dt, seed=sum(t))
    # a bias comparable to the outputs, so it moves the ReLU decisions
    bias = wl.quantize(wl.draw(("normal", 4.0), (sh.outC,), (77, sum(t), 0)), "f32")
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding, sh.outC,
                      DT_CODE[dt])
    x, w, b = dev(ops["x"]), dev(ops["w"]), dev(bias)
    fused = torch.empty(sh.y_shape(), dtype=torch.float32, device="cuda")
    names = _launch_names(lambda: pl.forward_relu(x, w, b, y=fused, implicit=implicit))
    # the forward GEMM's plan is the one d4r_gemm makes for (O, Kc, N)
    splits = d4r.d4r_gemm_workspace_size(sh.outC, pl.Kc, pl.N, 0, DT_CODE[dt]) > 0
    assert any(n.startswith("splitk_reduce:fwd") for n in names) == splits, names
    if t == CONV[-1]:
        assert splits
    plain = pl.forward_implicit(x, w, b) if implicit else pl.forward(x, w, b)
    d4r.d4r_relu_forward(plain, plain, plain.numel())
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    ref = oracle.relu(oracle.conv_forward(ops["x"].exact, ops["w"].exact, bias.exact, sh.stride, sh.padding))
    got = host(fused)
    assert (got >= 0).all()
    assert 0.2 < np.mean(got > 0) < 0.8  # the ReLU cut a real share of the outputs
    err = rel_err(got, ref)
    print(f"conv relu {t} {dt} implicit={implicit}: {err:.2e}", flush=True)
    assert err < TOL[dt], err


def test_conv_forward_relu_keeps_col_for_filter_gradient():
    # without D4R_FWD_IMPLICIT the fused forward leaves col in ws, so the
    # filter gradient with reuse_col = 1 equals the one from x
    sh = wl.ConvShape(2, 16, 9, 11, 3, 3, 1, 1, 40)
    ops = wl.random_conv(sh, "f32", seed=3)
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, 3, 3, 1, 1, sh.outC, d4r.D4R_F32)
    x, w, g, b = dev(ops["x"]), dev(ops["w"]), dev(ops["g"]), dev(ops["bias"])
    pl.forward_relu(x, w, b)
    dw_col, db_col = pl.backward_filter(None, g, reuse_col=True)
    dw_x, db_x = pl.backward_filter(x, g, reuse_col=False)
    torch.cuda.synchronize()
    assert torch.equal(dw_col, dw_x)
    assert torch.equal(db_col, db_x)


# (M, K, N): ragged small layers, LeNet's fc1, and a long K that splits in
# every dtype (f32 also splits the small ones: few tiles)
GEMM = [(5, 84, 10), (64, 256, 120), (37, 120, 84), (130, 96, 259), (24, 20000, 40), (24, 16, 70)]


def _gemm_case(M, K, N, flags, dt, seed):
    a = wl.draw(("normal", 1.0), (M, K), (88, seed, 1))
    bm = wl.draw(("normal", 1.0), (K, N), (88, seed, 2))
    bias = wl.draw(("normal", 0.5 * np.sqrt(K)), (N,), (88, seed, 3))
    A = wl.quantize(np.ascontiguousarray(a.T if flags & 1 else a), dt)
    Bm = wl.quantize(np.ascontiguousarray(bm.T if flags & 2 else bm), dt)
    return A, Bm, wl.quantize(bias, "f32")


@pytest.mark.parametrize("mkn", GEMM, ids=str)
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_gemm_bias_act(mkn, flags, dt):
    M, K, N = mkn
    A, Bm, bias = _gemm_case(M, K, N, flags, dt, seed=M + K + N + flags)
    code = DT_CODE[dt]
    wsb = d4r.d4r_gemm_workspace_size(M, K, N, flags, code)
    if K == 20000:
        assert wsb > 0
    if K == 16:
        assert wsb == 0
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    a, b, bb = dev(A), dev(Bm), dev(bias)
    out = {}
    for relu in (0, 1):
        out[relu] = torch.empty((M, N), dtype=torch.float32, device="cuda")
        names = _launch_names(lambda: d4r.d4r_gemm_bias_act(M, K, N, flags, code, a, b, bb, relu, out[relu],
                                                            ws, wsb))
        assert any(n.startswith("splitk_reduce:gemm_bias") for n in names) == (wsb > 0), names
    nob = torch.empty((M, N), dtype=torch.float32, device="cuda")
    d4r.d4r_gemm_bias_act(M, K, N, flags, code, a, b, None, 0, nob, ws, wsb)
    plain = torch.empty((M, N), dtype=torch.float32, device="cuda")
    d4r.d4r_gemm(M, K, N, flags, code, a, b, plain, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(nob, plain)
    d4r.d4r_add_bias_rows(plain, bb, plain, M, N)
    torch.cuda.synchronize()
    assert torch.equal(out[0], plain)
    d4r.d4r_relu_forward(plain, plain, plain.numel())
    torch.cuda.synchronize()
    assert torch.equal(out[1], plain)
    lin = oracle.add_bias_rows(oracle.gemm(A.exact, Bm.exact, M, K, N, flags), bias.exact)
    assert rel_err(host(out[0]), lin) < TOL[dt]
    got = host(out[1])
    assert 0.2 < np.mean(got > 0) < 0.8
    err = rel_err(got, oracle.relu(lin))
    print(f"gemm bias relu {mkn} flags={flags} {dt}: {err:.2e}", flush=True)
    assert err < TOL[dt], err
