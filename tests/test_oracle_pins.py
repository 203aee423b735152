"""Pins of the CPU oracle against things other than itself.

The pages print no worked numeric example for convolution or GEMM, so the
oracle is pinned by closed forms, special cases that reduce to library
routines, identities that any correct convolution satisfies, brute force on
tiny shapes and hand-worked fixtures under tests/golden/.  Each check is
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, a wrong stride or padding offset) fails it.

Sources: directcompute-nn page, "Convolution: The im2col Approach"
(forward / backward decomposition, bias semantics) and "Transpose via Flags"
(the two operand index formulas).
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.signal
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

rng = np.random.default_rng(12345)


def _rand(*shape):
    return rng.normal(size=shape)


def _shapes_tiny():
    # (B, C, H, W, O, kH, kW, s, p) -- includes non-square kernels, strides
    # up to 4, padding >= kernel and single-pixel outputs.
    return [
        (1, 1, 5, 5, 1, 3, 3, 1, 0),
        (2, 3, 7, 6, 2, 3, 2, 1, 1),
        (2, 2, 7, 7, 3, 5, 5, 2, 2),
        (1, 3, 6, 7, 2, 2, 3, 3, 1),
        (2, 1, 7, 5, 2, 1, 1, 4, 0),
        (1, 2, 4, 4, 2, 2, 2, 1, 3),   # p > k
        (2, 2, 3, 3, 1, 3, 3, 1, 0),   # 1x1 output
        (1, 3, 7, 7, 2, 5, 3, 4, 2),
        (2, 2, 5, 6, 3, 1, 2, 2, 1),
    ]


def _torch_conv(x, w, b, s, p):
    return torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w),
                                      None if b is None else torch.from_numpy(b),
                                      stride=s, padding=p).numpy()


def _rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def test_forward_1x1_is_matmul(orc):
    """1x1 stride-1 pad-0 conv: y[b] = W(O x C) @ x[b](C x HW) + bias."""
    B, C, H, W, O = 3, 5, 4, 6, 7
    x, w, bias = _rand(B, C, H, W), _rand(O, C, 1, 1), _rand(O)
    y = orc.conv_forward(x, w, bias, 1, 0)
    ref = np.stack([w[:, :, 0, 0] @ x[b].reshape(C, H * W) for b in range(B)])
    ref = ref.reshape(B, O, H, W) + bias[None, :, None, None]
    assert _rel(y, ref) < 1e-14


@pytest.mark.parametrize("k,s,p,u0,v0", [(3, 1, 1, 1, 1), (3, 1, 0, 2, 0),
                                          (5, 2, 2, 0, 4), (4, 3, 1, 3, 1),
                                          (11, 4, 2, 5, 7)])
def test_forward_delta_kernel_is_shift(orc, k, s, p, u0, v0):
    """W[o,c,u,v] = [o=c][u=u0][v=v0] gives y[b,o,i,j] = xt(b,o,i*s-p+u0, j*s-p+v0)."""
    B, C, H, W = 2, 3, 13, 17
    x = _rand(B, C, H, W)
    w = np.zeros((C, C, k, k))
    for c in range(C):
        w[c, c, u0, v0] = 1.0
    y = orc.conv_forward(x, w, None, s, p)
    OH, OW = y.shape[2:]
    xp = np.pad(x, ((0, 0), (0, 0), (p, p + k), (p, p + k)))
    ref = xp[:, :, u0:u0 + s * OH:s, v0:v0 + s * OW:s][:, :, :OH, :OW]
    assert np.array_equal(y, ref)
    if s == 1 and p == u0 == v0 and 2 * p + 1 == k:
        assert np.array_equal(y, x)  # identity


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_forward_matches_torch_f64(orc, shape):
    B, C, H, W, O, kH, kW, s, p = shape
    x, w, bias = _rand(B, C, H, W), _rand(O, C, kH, kW), _rand(O)
    y = orc.conv_forward(x, w, bias, s, p)
    assert _rel(y, _torch_conv(x, w, bias, s, p)) < 1e-13


@pytest.mark.parametrize("s", [1, 2, 3])
def test_forward_matches_scipy_correlate(orc, s):
    """Cross-correlation of the zero-padded plane, subsampled by the stride."""
    B, C, H, W, O, kH, kW, p = 2, 3, 9, 8, 2, 3, 4, 2
    x, w = _rand(B, C, H, W), _rand(O, C, kH, kW)
    y = orc.conv_forward(x, w, None, s, p)
    OH, OW = y.shape[2:]
    ref = np.zeros_like(y)
    for b in range(B):
        for o in range(O):
            acc = 0
            for c in range(C):
                xp = np.pad(x[b, c], p)
                acc = acc + scipy.signal.correlate2d(xp, w[o, c], mode="valid")
            ref[b, o] = acc[::s, ::s][:OH, :OW]
    assert _rel(y, ref) < 1e-13


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", _shapes_tiny())
def test_backward_matches_torch_autograd_f64(orc, shape):
    B, C, H, W, O, kH, kW, s, p = shape
    x, w, bias = _rand(B, C, H, W), _rand(O, C, kH, kW), _rand(O)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    bt = torch.from_numpy(bias).requires_grad_()
    yt = torch.nn.functional.conv2d(xt, wt, bt, stride=s, padding=p)
    g = _rand(*yt.shape)
    yt.backward(torch.from_numpy(g))
    dx = orc.conv_backward_data(g, w, x.shape, s, p)
    dw = orc.conv_backward_filter(x, g, w.shape, s, p)
    db = orc.conv_backward_bias(g)
    assert _rel(dx, xt.grad.numpy()) < 1e-13
    assert _rel(dw, wt.grad.numpy()) < 1e-13
    assert _rel(db, bt.grad.numpy()) < 1e-13


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_adjoint_identities(orc, shape):
    """<y - bias, g> = <x, dx> = <W, dW>  and  <db, 1> = sum(g)."""
    B, C, H, W, O, kH, kW, s, p = shape
    x, w, bias = _rand(B, C, H, W), _rand(O, C, kH, kW), _rand(O)
    y = orc.conv_forward(x, w, bias, s, p)
    g = _rand(*y.shape)
    dx = orc.conv_backward_data(g, w, x.shape, s, p)
    dw = orc.conv_backward_filter(x, g, w.shape, s, p)
    db = orc.conv_backward_bias(g)
    lhs = np.vdot(y - bias[None, :, None, None], g)
    scale = np.abs(y).sum() * np.abs(g).max() + 1.0
    assert abs(lhs - np.vdot(x, dx)) / scale < 1e-12
    assert abs(lhs - np.vdot(w, dw)) / scale < 1e-12
    assert abs(db.sum() - g.sum()) < 1e-10
    assert np.allclose(db, g.sum(axis=(0, 2, 3)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(1, 2, 4, 5, 2, 3, 2, 1, 1), (2, 1, 5, 5, 2, 3, 3, 2, 2),
                                   (1, 2, 6, 4, 1, 2, 2, 3, 0)])
def test_toeplitz_brute_force(orc, shape):
    """Build the dense matrices of the forward map (linear in x for fixed W,
    and in W for fixed x) from unit inputs; dx and dW must be their
    transposes applied to g.  This checks the backward loops against the
    forward definition alone."""
    B, C, H, W, O, kH, kW, s, p = shape
    x, w = _rand(B, C, H, W), _rand(O, C, kH, kW)
    OH, OW = orc.out_dims(H, W, kH, kW, s, p)
    g = _rand(B, O, OH, OW)
    Tx = np.zeros((g.size, x.size))
    for e in range(x.size):
        ex = np.zeros(x.size)
        ex[e] = 1.0
        Tx[:, e] = orc.conv_forward(ex.reshape(x.shape), w, None, s, p).ravel()
    Tw = np.zeros((g.size, w.size))
    for e in range(w.size):
        ew = np.zeros(w.size)
        ew[e] = 1.0
        Tw[:, e] = orc.conv_forward(x, ew.reshape(w.shape), None, s, p).ravel()
    # the two dense maps agree on the forward itself
    y = orc.conv_forward(x, w, None, s, p).ravel()
    assert np.allclose(Tx @ x.ravel(), y, atol=1e-12)
    assert np.allclose(Tw @ w.ravel(), y, atol=1e-12)
    dx = orc.conv_backward_data(g, w, x.shape, s, p).ravel()
    dw = orc.conv_backward_filter(x, g, w.shape, s, p).ravel()
    assert np.allclose(dx, Tx.T @ g.ravel(), atol=1e-12)
    assert np.allclose(dw, Tw.T @ g.ravel(), atol=1e-12)


def test_finite_differences_f64(orc):
    """Central differences of L = <conv(x; W, b), g> against dx, dW, db.
    L is linear in each argument, so the difference quotient is exact up to
    rounding."""
    B, C, H, W, O, kH, kW, s, p = 2, 2, 5, 6, 3, 3, 2, 2, 1
    x, w, bias = _rand(B, C, H, W), _rand(O, C, kH, kW), _rand(O)
    y = orc.conv_forward(x, w, bias, s, p)
    g = _rand(*y.shape)
    L = lambda xx, ww, bb: float(np.vdot(orc.conv_forward(xx, ww, bb, s, p), g))
    h = 1e-3
    dx = orc.conv_backward_data(g, w, x.shape, s, p)
    dw = orc.conv_backward_filter(x, g, w.shape, s, p)
    db = orc.conv_backward_bias(g)
    for arr, grad, which in ((x, dx, 0), (w, dw, 1), (bias, db, 2)):
        for idx in np.ndindex(arr.shape):
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = [x, w, bias]
            args_m = [x, w, bias]
            args_p[which], args_m[which] = plus, minus
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-9 * max(1.0, abs(grad[idx])), (which, idx)


def test_bias_grad_closed_form(orc):
    g = _rand(3, 4, 5, 6)
    db = orc.conv_backward_bias(g)
    for o in range(4):
        assert abs(db[o] - sum(float(v) for v in g[:, o].ravel())) < 1e-12


# --------------------------------------------------------------------------
# GEMM with transpose flags
# --------------------------------------------------------------------------

@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (7, 17, 5), (16, 63, 65), (6, 25, 33)])
def test_gemm_flags_match_numpy(orc, flags, M, K, N):
    """flags&1: A stored K x M (transposed); flags&2: B stored N x K."""
    a, b = _rand(M, K), _rand(K, N)
    a_st = a.T.copy() if flags & 1 else a
    b_st = b.T.copy() if flags & 2 else b
    c = orc.gemm(a_st, b_st, M, K, N, flags)
    assert _rel(c, a @ b) < 1e-14


def test_gemm_rejects_bad_flags(orc):
    with pytest.raises(ValueError):
        orc.gemm(np.ones(4), np.ones(4), 2, 2, 2, 4)


# --------------------------------------------------------------------------
# Index-map specifications (im2col / col2im)
# --------------------------------------------------------------------------

def _coverage(n, k, s, p):
    """Closed form, counted over output positions i (not kernel taps u):
    input row h is read by i in [ceil((h+p-k+1)/s), floor((h+p)/s)] within [0, out)."""
    out = (n + 2 * p - k) // s + 1
    cnt = np.zeros(n, dtype=np.int64)
    for h in range(n):
        lo = max(0, -((-(h + p - k + 1)) // s))
        hi = min(out - 1, (h + p) // s)
        cnt[h] = max(0, hi - lo + 1)
    return cnt


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_im2col_spec_times_filters_is_conv(orc, shape):
    """Wmat @ im2col(x), reshaped, equals the direct-loop conv (the method's
    forward reaches the definition)."""
    B, C, H, W, O, kH, kW, s, p = shape
    x, w = _rand(B, C, H, W), _rand(O, C, kH, kW)
    col = orc.im2col_spec(x, kH, kW, s, p)
    OH, OW = orc.out_dims(H, W, kH, kW, s, p)
    cm = w.reshape(O, -1) @ col
    y = cm.reshape(O, B, OH, OW).transpose(1, 0, 2, 3)
    assert _rel(y, _torch_conv(x, w, None, s, p)) < 1e-13


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_im2col_spec_iota_codes(orc, shape):
    """With x[k] = k+1 every col entry is its source's code or 0 (padding),
    and each code appears cnt_h(h)*cnt_w(w) times."""
    B, C, H, W, O, kH, kW, s, p = shape
    x = np.arange(1, B * C * H * W + 1, dtype=np.float64).reshape(B, C, H, W)
    col = orc.im2col_spec(x, kH, kW, s, p)
    assert np.all(col == np.round(col))
    counts = np.bincount(col.astype(np.int64).ravel(), minlength=x.size + 1)[1:]
    expect = np.outer(_coverage(H, kH, s, p), _coverage(W, kW, s, p))
    assert np.array_equal(counts.reshape(B, C, H, W), np.broadcast_to(expect, (B, C, H, W)))
    OH, OW = orc.out_dims(H, W, kH, kW, s, p)
    # every col entry has the code of the source element the formula names
    for r, n in itertools.product(range(col.shape[0]), range(0, col.shape[1], 3)):
        c, u, v = r // (kH * kW), (r // kW) % kH, r % kW
        b, i, j = n // (OH * OW), (n // OW) % OH, n % OW
        h, ww = i * s - p + u, j * s - p + v
        want = x[b, c, h, ww] if 0 <= h < H and 0 <= ww < W else 0.0
        assert col[r, n] == want


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_col2im_spec_coverage_and_adjoint(orc, shape):
    B, C, H, W, O, kH, kW, s, p = shape
    OH, OW = orc.out_dims(H, W, kH, kW, s, p)
    R, N = C * kH * kW, B * OH * OW
    ones = orc.col2im_spec(np.ones((R, N)), (B, C, H, W), kH, kW, s, p)
    expect = np.outer(_coverage(H, kH, s, p), _coverage(W, kW, s, p))
    assert np.array_equal(ones, np.broadcast_to(expect, ones.shape).astype(np.float64))
    # adjoint, exact with small integers
    r2 = np.random.default_rng(7)
    x = r2.integers(-8, 9, size=(B, C, H, W)).astype(np.float64)
    c = r2.integers(-8, 9, size=(R, N)).astype(np.float64)
    assert np.vdot(orc.im2col_spec(x, kH, kW, s, p), c) == \
        np.vdot(x, orc.col2im_spec(c, (B, C, H, W), kH, kW, s, p))


@pytest.mark.parametrize("shape", _shapes_tiny())
def test_col2im_of_wt_g_is_data_grad(orc, shape):
    """col2im(W^T G) equals the direct-loop data gradient."""
    B, C, H, W, O, kH, kW, s, p = shape
    w = _rand(O, C, kH, kW)
    OH, OW = orc.out_dims(H, W, kH, kW, s, p)
    g = _rand(B, O, OH, OW)
    G = g.transpose(1, 0, 2, 3).reshape(O, -1)
    dcol = w.reshape(O, -1).T @ G
    dx = orc.col2im_spec(dcol, (B, C, H, W), kH, kW, s, p)
    assert _rel(dx, orc.conv_backward_data(g, w, (B, C, H, W), s, p)) < 1e-13


# --------------------------------------------------------------------------
# Hand-worked fixtures and error behaviour
# --------------------------------------------------------------------------

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(GOLDEN)
                                        if f.startswith("conv_") and f.endswith(".json")))
def test_golden_conv_fixture(orc, name):
    d = _golden(name)
    x, w = np.array(d["x"], float), np.array(d["w"], float)
    bias = np.array(d["bias"], float) if d.get("bias") is not None else None
    s, p = d["stride"], d["padding"]
    y = orc.conv_forward(x, w, bias, s, p)
    assert np.array_equal(y, np.array(d["y"], float))
    if "g" in d:
        g = np.array(d["g"], float)
        assert np.array_equal(orc.conv_backward_data(g, w, x.shape, s, p), np.array(d["dx"], float))
        assert np.array_equal(orc.conv_backward_filter(x, g, w.shape, s, p), np.array(d["dw"], float))
        assert np.array_equal(orc.conv_backward_bias(g), np.array(d["db"], float))


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(GOLDEN)
                                        if f.startswith("gemm_") and f.endswith(".json")))
def test_golden_gemm_fixture(orc, name):
    d = _golden(name)
    c = orc.gemm(np.array(d["A"], float), np.array(d["B"], float),
                 d["M"], d["K"], d["N"], d["flags"])
    assert np.array_equal(c, np.array(d["C"], float))


def test_invalid_geometry_rejected(orc):
    with pytest.raises(ValueError):
        orc.conv_forward(np.ones((1, 1, 2, 2)), np.ones((1, 1, 5, 5)), None, 1, 0)
    with pytest.raises(ValueError):
        orc.conv_forward(np.ones((1, 2, 4, 4)), np.ones((1, 1, 3, 3)), None, 1, 0)
    with pytest.raises(ValueError):
        orc.out_dims(4, 4, 3, 3, 0, 0)
