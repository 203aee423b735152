"""GPU parity of the combined backward (d4r_conv_backward).

Where the layer takes the NHWC data gradient and copies dy for the filter
gradient, one launch reads dy once and writes both GEMM operands (G and its
NHWC transpose) and the bias partial sums, with the filter flip in the same
launch.  dx and dw must then equal the two separate calls bit for bit (same
operands, same GEMMs); db differs from the separate path only in summation
order, so it is checked against the oracle and for run-to-run equality.
Shapes where the fused preparation does not apply must give exactly the
separate calls, except f32 layers with an explicit data gradient (dcol +
col2im) and at least 32 output channels: there the combined call reshapes
dy once into G for both GEMMs.  Its dx must still equal the separate call's
bit for bit (same plan and kernel; the operands reach the MFMAs as the same
fragments in the same k order); dw and db
come from other kernels or another summation order, so they are checked
against the oracle and for run-to-run equality.  Which path ran is read from
the profile recorder and the plan description.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

# (batch, C, H, W, kH, kW, stride, pad, O), {dtypes where dy is prepared in one pass}
SHAPES = [
    ((2, 128, 7, 9, 3, 3, 1, 1, 64), {"f32", "f16", "bf16"}),   # C*k*k = 1152: f32 copies dy too
    ((3, 64, 13, 13, 3, 3, 1, 1, 128), {"f16", "bf16"}),         # P = 169: three pixel tiles
    ((1, 32, 20, 20, 5, 5, 1, 2, 64), {"f16", "bf16"}),
    ((2, 16, 9, 9, 3, 3, 2, 1, 64), set()),                      # stride 2: explicit data gradient
    ((3, 3, 23, 23, 5, 5, 4, 2, 40), set()),                     # stride 4, 3 channels (AlexNet conv1-like)
    ((2, 64, 9, 9, 3, 3, 2, 1, 64), set()),                      # stride 2: phased data gradient
    ((2, 16, 5, 7, 1, 1, 1, 0, 64), set()),                      # 1x1: direct path
    ((2, 32, 8, 8, 3, 3, 1, 1, 40), set()),                      # O not a whole GEMM stage
    ((1, 128, 1, 1, 3, 3, 1, 1, 64), {"f32", "f16", "bf16"}),    # one output pixel (P = 1)
    ((3, 128, 2, 5, 3, 3, 1, 1, 128), {"f32", "f16", "bf16"}),   # P = 10: one partial pixel tile per image
    # padding above kH - 1: the NHWC data gradient with a negative flipped padding
    ((2, 32, 6, 6, 2, 2, 1, 3, 64), {"f16", "bf16"}),
    ((1, 64, 5, 5, 3, 3, 1, 3, 128), {"f16", "bf16"}),
]


def _names(fn):
    d4r.d4r_profile_reset()
    d4r.d4r_profile_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
        return [r["name"] for r in d4r.d4r_profile_read()]
    finally:
        d4r.d4r_profile_enable(False)
        d4r.d4r_profile_reset()


def _plan(sh, dt):
    return d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding, sh.outC,
                        DT_CODE[dt])


@pytest.mark.parametrize("t,fused_dts", SHAPES, ids=[str(s[0]) for s in SHAPES])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("reuse_col", [True, False])
def test_combined_backward(t, fused_dts, dt, reuse_col):
    sh = wl.ConvShape(*t)
    ops = wl.random_conv(sh, dt, seed=sum(t) + 5)
    x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl = _plan(sh, dt)
    if reuse_col:
        pl.forward(x, w)
    out = {}

    def run():
        out["c"] = pl.backward(x, w, g, reuse_col=reuse_col)

    names = _names(run)
    assert any(n.startswith("dy_prep_") for n in names) == (dt in fused_dts), names
    explicit = pl.describe()["fused_backward"] == "explicit"
    if explicit:
        # one pass over dy: no transposed copy of it, no in-place bias pass
        assert sum(n.startswith("grad_reshape") for n in names) == 1, names
        assert not any("dgrad_dy" in n or n.startswith("bias_partial") for n in names), names
    dx, dw, db = out["c"]
    # the separate calls on the same inputs
    ref_dx = pl.backward_data_implicit(w, g)
    if reuse_col:
        pl.forward(x, w)
    ref_dw, ref_db = pl.backward_filter(x, g, reuse_col=reuse_col)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref_dx)
    if not explicit:
        assert torch.equal(dw, ref_dw)
    if dt not in fused_dts and not explicit:
        assert torch.equal(db, ref_db)
    # again: run-to-run identical
    if reuse_col:
        pl.forward(x, w)
    dx2, dw2, db2 = pl.backward(x, w, g, reuse_col=reuse_col)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx) and torch.equal(dw2, dw) and torch.equal(db2, db)
    # the oracle
    X, Wt, G = ops["x"].exact, ops["w"].exact, ops["g"].exact
    s, p = sh.stride, sh.padding
    refs = {"dx": (host(dx), oracle.conv_backward_data(G, Wt, sh.x_shape(), s, p)),
            "dw": (host(dw), oracle.conv_backward_filter(X, G, sh.w_shape(), s, p)),
            "db": (host(db), oracle.conv_backward_bias(G))}
    for k, (got, ref) in refs.items():
        err = rel_err(got, ref)
        print(f"combined backward {t} {dt} reuse={reuse_col} {k}: {err:.2e}", flush=True)
        assert err < TOL[dt], (k, err)


def test_combined_backward_without_bias():
    sh = wl.ConvShape(2, 128, 7, 9, 3, 3, 1, 1, 64)
    ops = wl.random_conv(sh, "bf16", seed=11)
    x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl = _plan(sh, "bf16")
    dx, dw, db = pl.backward(x, w, g, reuse_col=False, want_bias=False)
    ref_dw, _ = pl.backward_filter(x, g, reuse_col=False, want_bias=False)
    torch.cuda.synchronize()
    assert db is None
    assert torch.equal(dw, ref_dw)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_combined_backward_alexnet_conv4_full_size(dt):
    # the bench's layer at its real shape: dx and dw against the separate
    # calls (checked against the oracle by the full-size parity tests), db
    # against the oracle over the whole batch
    w_ = wl.WORKLOADS["c4"]
    sh = w_.layers[1].shape
    ops = wl.conv_inputs(w_, 1, dt)
    x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl = _plan(sh, dt)
    pl.forward(x, w)
    names = _names(lambda: pl.backward(None, w, g, reuse_col=True))
    assert any(n.startswith("dy_prep_") for n in names), names
    pl.forward(x, w)
    dx, dw, db = pl.backward(None, w, g, reuse_col=True)
    ref_dx = pl.backward_data_implicit(w, g)
    ref_dw, _ = pl.backward_filter(x, g, reuse_col=False)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref_dx)
    assert torch.equal(dw, ref_dw)
    err = rel_err(host(db), oracle.conv_backward_bias(ops["g"].exact))
    assert err < TOL[dt], err


# f32 layers with an explicit data gradient: the combined call's one-pass
# form (on by default from 32 output channels) against the separate calls,
# with the switch forced either way and with the transposed-W variant
EXPLICIT_SHAPES = [
    (3, 3, 23, 23, 5, 5, 4, 2, 40),     # stride 4, 3 channels (AlexNet conv1-like)
    (2, 16, 9, 9, 3, 3, 2, 1, 64),      # stride 2, too few channels for the phased form
    (2, 5, 11, 9, 3, 2, 2, 1, 33),      # ragged: O, Kc and N off every tile
    (1, 3, 12, 12, 4, 4, 3, 0, 8),      # few output channels: separate calls by default
]


@pytest.mark.parametrize("t", EXPLICIT_SHAPES, ids=[str(s) for s in EXPLICIT_SHAPES])
@pytest.mark.parametrize("mode", ["default", "off", "on", "on_rows"])
def test_combined_backward_explicit_one_pass(t, mode, monkeypatch):
    env = {"off": {"D4R_FUSED_EXPLICIT": "0"}, "on": {"D4R_FUSED_EXPLICIT": "1"},
           "on_rows": {"D4R_FUSED_EXPLICIT": "1", "D4R_FX_WT": "0"}}.get(mode, {})
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    sh = wl.ConvShape(*t)
    ops = wl.random_conv(sh, "f32", seed=sum(t) + 17)
    x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl = _plan(sh, "f32")
    d = pl.describe()
    want = {"default": sh.outC >= 32, "off": False}.get(mode, True)
    assert (d["fused_backward"] == "explicit") == want, d
    assert d.get("fx_wt") == (None if not want else "0" if mode == "on_rows" else "1")
    out = {}
    names = _names(lambda: out.setdefault("c", pl.backward(x, w, g, reuse_col=False)))
    assert any(n.startswith("grad_reshape") for n in names) == want, names
    dx, dw, db = out["c"]
    ref_dx = pl.backward_data_implicit(w, g)
    torch.cuda.synchronize()
    # W, row-contiguous or transposed, and dy, in place or reshaped, reach
    # the MFMAs as the same fragments in the same k order
    assert torch.equal(dx, ref_dx)
    dx2, dw2, db2 = pl.backward(x, w, g, reuse_col=False)
    torch.cuda.synchronize()
    assert torch.equal(dx2, dx) and torch.equal(dw2, dw) and torch.equal(db2, db)
    X, Wt, G = ops["x"].exact, ops["w"].exact, ops["g"].exact
    s, p = sh.stride, sh.padding
    for k, got, ref in [("dx", dx, oracle.conv_backward_data(G, Wt, sh.x_shape(), s, p)),
                        ("dw", dw, oracle.conv_backward_filter(X, G, sh.w_shape(), s, p)),
                        ("db", db, oracle.conv_backward_bias(G))]:
        err = rel_err(host(got), ref)
        print(f"explicit one-pass backward {t} {mode} {k}: {err:.2e}", flush=True)
        assert err < TOL["f32"], (k, err)
