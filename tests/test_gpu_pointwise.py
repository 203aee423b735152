"""GPU parity of the direct path of 1x1, stride-1, unpadded convolutions.

For such a convolution the col matrix is x with the batch folded into its
columns, so the library's GEMMs read x and dy where they lie (NCHW): the
implicit forward is W * x[b], the data gradient W^T * dy[b] stored straight
into dx (no dcol, no col2im), and the filter gradient without a saved col
sums dy[b] * x[b]^T (no im2col).  Every entry point is checked against the
oracle's direct convolution, in each dtype, on pixel counts that are and are
not multiples of 8 (16-byte vectors or single-element loads), with images
straddling tiles and split K; the im2col path (D4R_POINTWISE=0) must agree.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu

# (batch, C, H, W, O): P = 35 (ragged), 64, 24 with O > 128, a single pixel,
# C = 1, and one image with P = 3680 (the 46x80 map) at reduced channels
SHAPES = [(2, 16, 5, 7, 24), (3, 64, 8, 8, 40), (2, 8, 4, 6, 130), (5, 3, 1, 1, 7), (4, 1, 6, 6, 9),
          (1, 32, 46, 80, 16)]


def _inputs(t, dt):
    B, C, H, W, O = t
    sh = wl.ConvShape(B, C, H, W, 1, 1, 1, 0, O)
    return sh, wl.random_conv(sh, dt, seed=B * 7 + C + O)


def _run_all(sh, dt, ops):
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, 1, 1, 1, 0, sh.outC, DT_CODE[dt])
    x, w, g, bias = dev(ops["x"]), dev(ops["w"]), dev(ops["g"]), dev(ops["bias"])
    out = {}
    out["y_impl"] = pl.forward_implicit(x, w, bias)
    out["dx"] = pl.backward_data(w, g)
    out["dx_impl"] = pl.backward_data_implicit(w, g)
    out["dw"], out["db"] = pl.backward_filter(x, g, reuse_col=False)
    out["y"] = pl.forward(x, w, bias)                        # im2col + GEMM, col saved
    out["dw_col"], out["db_col"] = pl.backward_filter(None, g, reuse_col=True)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


@pytest.mark.parametrize("t", SHAPES, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_pointwise_entry_points_match_oracle(t, dt):
    sh, ops = _inputs(t, dt)
    got = _run_all(sh, dt, ops)
    ry = oracle.conv_forward(ops["x"].exact, ops["w"].exact, ops["bias"].exact, 1, 0)
    rdx = oracle.conv_backward_data(ops["g"].exact, ops["w"].exact, sh.x_shape(), 1, 0)
    rdw = oracle.conv_backward_filter(ops["x"].exact, ops["g"].exact, sh.w_shape(), 1, 0)
    rdb = oracle.conv_backward_bias(ops["g"].exact)
    refs = {"y": ry, "y_impl": ry, "dx": rdx, "dx_impl": rdx, "dw": rdw, "dw_col": rdw, "db": rdb,
            "db_col": rdb}
    for k, ref in refs.items():
        err = rel_err(got[k], ref)
        print(f"pointwise {t} {dt} {k}: {err:.2e}", flush=True)
        assert err < TOL[dt], (t, dt, k, err)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_pointwise_matches_im2col_path(dt, monkeypatch):
    sh, ops = _inputs((3, 64, 8, 8, 40), dt)
    direct = _run_all(sh, dt, ops)
    monkeypatch.setenv("D4R_POINTWISE", "0")
    via_col = _run_all(sh, dt, ops)
    for k in direct:
        assert rel_err(direct[k], via_col[k]) < TOL[dt], k


def test_pointwise_feature_map_layer_full_size():
    # the 46x80 map's 1x1 256 -> 128 layer at its real shape (batch 4, f16):
    # the data gradient (no dcol) and the direct filter gradient on sampled
    # channels the oracle computes exactly
    w = wl.WORKLOADS["c5"]
    li = [l.name for l in w.layers].index("conv1x1")
    sh = w.layers[li].shape
    ops = wl.conv_inputs(w, li, "f16")
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, 1, 1, 1, 0, sh.outC, d4r.D4R_F16)
    x, wt, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    dx = pl.backward_data(wt, g)
    dw, db = pl.backward_filter(x, g, reuse_col=False)
    y = pl.forward_implicit(x, wt, dev(ops["bias"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    cs = np.sort(rng.choice(sh.inC, 8, replace=False))
    os_ = np.sort(rng.choice(sh.outC, 8, replace=False))
    X, Wt, G, bias = ops["x"].exact, ops["w"].exact, ops["g"].exact, ops["bias"].exact
    # sampled channels: each is a whole smaller convolution for the oracle
    rdx = oracle.conv_backward_data(G, Wt[:, cs], (sh.batch, len(cs), sh.inH, sh.inW), 1, 0)
    rdw = oracle.conv_backward_filter(X[:, cs], G[:, os_], (len(os_), len(cs), 1, 1), 1, 0)
    ry = oracle.conv_forward(X, Wt[os_], bias[os_], 1, 0)
    assert rel_err(host(dx)[:, cs], rdx) < TOL["f16"]
    assert rel_err(host(dw)[os_][:, cs], rdw) < TOL["f16"]
    assert rel_err(host(y)[:, os_], ry) < TOL["f16"]
    assert rel_err(host(db), oracle.conv_backward_bias(G)) < TOL["f16"]
