"""GPU parity: libd4r_conv (through its C ABI) against the CPU oracle.

* im2col and col2im index maps: bit-exact against the oracle's index-map
  specifications (iota codes, raw 16-bit patterns, small-integer dcol).
* GEMM with flags 0..3 in f32 / f16 / bf16 on odd shapes.
* Whole-tensor parity of forward, data, filter and bias gradients on every
  workload at a batch the oracle finishes in seconds (several tiles, ragged
  tails).
* Full-size parity (the bench's launch configuration) on sampled channel /
  image blocks, which the oracle computes exactly because y[b, o] depends
  only on x[b] and W[o], dx[b, c] only on dy[b] and W[:, c], and dW[o, c]
  only on x[:, c] and dy[:, o].
Tolerances: relative Frobenius error 1e-5 (f32), 2e-3 (f16 / bf16 inputs
with f32 accumulation).
"""
import sys

import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import DT_CODE, TOL, bits16, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


TINY = [
    # (B, C, H, W, O, kH, kW, s, p)
    (1, 1, 5, 5, 1, 3, 3, 1, 0),
    (2, 3, 7, 6, 5, 3, 2, 1, 1),
    (2, 2, 7, 7, 3, 5, 5, 2, 2),
    (1, 3, 6, 7, 2, 2, 3, 3, 1),
    (3, 1, 7, 5, 2, 1, 1, 4, 0),
    (1, 2, 4, 4, 2, 2, 2, 1, 3),
    (2, 2, 3, 3, 1, 3, 3, 1, 0),
    (2, 5, 17, 19, 33, 3, 3, 1, 1),
    (3, 7, 23, 29, 65, 5, 3, 2, 2),
    (2, 17, 12, 12, 130, 3, 3, 1, 1),
]


def _shape(t):
    B, C, H, W, O, kH, kW, s, p = t
    return wl.ConvShape(B, C, H, W, kH, kW, s, p, O)


def _plan(sh: wl.ConvShape, dt: str) -> d4r.ConvPlan:
    return d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding,
                        sh.outC, DT_CODE[dt])


# ---------------------------------------------------------------------------
# index maps
# ---------------------------------------------------------------------------

def _im2col_cases():
    cases = [(_shape(t), dt) for t in TINY for dt in ("f32", "bf16")]
    for key, w in wl.WORKLOADS.items():
        for layer in w.layers:
            sh = layer.shape
            cases.append((sh.with_batch(min(sh.batch, 2)), w.dtypes[-1]))
    return cases


@pytest.mark.parametrize("sh,dt", _im2col_cases(), ids=lambda v: str(v))
def test_im2col_bit_exact(sh, dt):
    _say("im2col", sh, dt)
    n = int(np.prod(sh.x_shape()))
    codes = np.arange(1, n + 1, dtype=np.int64)
    if dt == "f32":
        assert n < 2 ** 24
        x = torch.from_numpy(codes.astype(np.float32).reshape(sh.x_shape())).cuda()
        ref = oracle.im2col_spec(codes.reshape(sh.x_shape()).astype(np.float64), sh.kH, sh.kW,
                                 sh.stride, sh.padding)
    else:
        pat = (codes * 2654435761) % 65521 + 1          # nonzero 16-bit patterns
        x = torch.from_numpy(pat.astype(np.uint16).view(np.int16).reshape(sh.x_shape())).cuda()
        x = x.view(torch.bfloat16 if dt == "bf16" else torch.float16)
        ref = oracle.im2col_spec(pat.reshape(sh.x_shape()).astype(np.float64), sh.kH, sh.kW,
                                 sh.stride, sh.padding)
    pl = _plan(sh, dt)
    col = torch.empty((sh.Kc, sh.N), dtype=x.dtype, device="cuda")
    d4r.d4r_conv_im2col(pl.h, x, col)
    torch.cuda.synchronize()
    if dt == "f32":
        got = col.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref)
    else:
        assert np.array_equal(bits16(col).astype(np.int64), ref.astype(np.int64))


# Stride-1 maps whose output width is a multiple of 8 take the shifted-copy
# im2col (8x8 with 256 channels: several images per block); the general
# LDS kernel must give the same bits with it switched off.
SHIFT_SHAPES = [(64, 256, 8, 8, 16, 3, 3, 1, 1), (3, 5, 6, 16, 4, 5, 5, 1, 2), (2, 4, 9, 24, 3, 1, 1, 1, 0),
                (4, 7, 10, 8, 2, 3, 3, 1, 1)]


@pytest.mark.parametrize("t", SHIFT_SHAPES, ids=str)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shift", ["1", "0"])
def test_im2col_shifted_copies_bit_exact(t, dt, shift, monkeypatch):
    monkeypatch.setenv("D4R_IM2COL_SHIFT", shift)
    test_im2col_bit_exact(_shape(t), dt)


@pytest.mark.parametrize("sh", [_shape(t) for t in TINY] +
                         [l.shape.with_batch(min(l.shape.batch, 2)) for w in wl.WORKLOADS.values()
                          for l in w.layers], ids=str)
def test_col2im_bit_exact(sh):
    _say("col2im", sh)
    rng = np.random.default_rng(31)
    dcol = rng.integers(-8, 9, size=(sh.Kc, sh.N)).astype(np.float32)
    ref = oracle.col2im_spec(dcol.astype(np.float64), sh.x_shape(), sh.kH, sh.kW, sh.stride, sh.padding)
    pl = _plan(sh, "f32")
    dx = torch.empty(sh.x_shape(), dtype=torch.float32, device="cuda")
    d4r.d4r_conv_col2im(pl.h, torch.from_numpy(dcol).cuda(), dx)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy().astype(np.float64), ref)


def test_col2im_coverage_closed_form():
    sh = wl.ConvShape(2, 3, 224, 224, 11, 11, 4, 2, 4)
    pl = _plan(sh, "f32")
    dx = torch.empty(sh.x_shape(), dtype=torch.float32, device="cuda")
    d4r.d4r_conv_col2im(pl.h, torch.ones((sh.Kc, sh.N), device="cuda"), dx)
    torch.cuda.synchronize()

    def cov(n, k, s, p):
        out = (n + 2 * p - k) // s + 1
        return np.array([max(0, min(out - 1, (h + p) // s) - max(0, -((-(h + p - k + 1)) // s)) + 1)
                         for h in range(n)])
    expect = np.outer(cov(224, 11, 4, 2), cov(224, 11, 4, 2))
    assert np.array_equal(dx.cpu().numpy()[1, 2], expect.astype(np.float32))


# ---------------------------------------------------------------------------
# GEMM with transpose flags
# ---------------------------------------------------------------------------

GEMM_SHAPES = [(1, 1, 1), (7, 17, 5), (16, 63, 65), (6, 25, 4608), (33, 129, 127),
               (64, 256, 120), (64, 120, 84), (130, 300, 257), (96, 1000, 363),
               (384, 72, 200), (257, 64, 129)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_parity(dt, flags, M, K, N):
    rng = np.random.default_rng(M * 1000003 + K * 101 + N + flags)
    a = wl.quantize(rng.normal(size=(K, M) if flags & 1 else (M, K)), dt)
    b = wl.quantize(rng.normal(size=(N, K) if flags & 2 else (K, N)), dt)
    ref = oracle.gemm(a.exact, b.exact, M, K, N, flags)
    C = d4r.gemm(dev(a), dev(b), M, K, N, flags)
    torch.cuda.synchronize()
    err = rel_err(host(C), ref)
    assert err < TOL[dt], err


def test_gemm_long_k_split_f32():
    """AlexNet conv1 filter-gradient shape: K = 96800 (split-K path)."""
    M, K, N = 96, 96800, 363
    rng = np.random.default_rng(5)
    a = wl.quantize(rng.normal(size=(M, K)), "f32")
    b = wl.quantize(rng.uniform(size=(N, K)), "f32")
    ref = oracle.gemm(a.exact, b.exact, M, K, N, 2)
    C = d4r.gemm(dev(a), dev(b), M, K, N, 2)
    torch.cuda.synchronize()
    err = rel_err(host(C), ref)
    _say("long-K f32 rel err", err)
    assert err < 1e-5


# ---------------------------------------------------------------------------
# whole-tensor conv parity
# ---------------------------------------------------------------------------

def _run_conv(sh, dt, ops):
    pl = _plan(sh, dt)
    x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    bias = dev(ops["bias"])
    y = pl.forward(x, w, bias)
    dx = pl.backward_data(w, g)
    dw, db = pl.backward_filter(None, g, reuse_col=True)
    torch.cuda.synchronize()
    return pl, y, dx, dw, db


def elementwise_bound(got, ref, aref, n_terms, what):
    """Per-element forward-error bound of float32 summation: every output is
    a sum of at most n_terms products (exact for 16-bit operands, one
    rounding each for float32), so |got - exact| <= gamma * sum |terms| with
    gamma = 2 (n_terms + 2) 2^-24 (a factor 2 over the textbook n u for
    accumulators that do not round to nearest).  aref is the oracle on the
    absolute values of the operands, i.e. sum |terms| per element.  A wrong
    or dropped block of terms leaves errors of order |y| >> gamma sum |terms|."""
    got = np.asarray(got, dtype=np.float64)
    bound = 2.0 * (n_terms + 2) * 2.0 ** -24 * np.asarray(aref, dtype=np.float64) + 1e-30
    viol = np.abs(got - ref) > bound
    assert not viol.any(), (what, int(viol.sum()), float(np.max(np.abs(got - ref) / bound)))


def _abs_refs(sh, X, Wt, G, bias):
    """The oracle on |x|, |W|, |g|, |bias|: sum of |terms| of every output."""
    s, p = sh.stride, sh.padding
    ax, aw, ag = np.abs(X), np.abs(Wt), np.abs(G)
    return (oracle.conv_forward(ax, aw, np.abs(bias), s, p),
            oracle.conv_backward_data(ag, aw, X.shape, s, p),
            oracle.conv_backward_filter(ax, ag, Wt.shape, s, p),
            oracle.conv_backward_bias(ag))


def _check_whole(sh, dt, ops, tag):
    _say("conv", tag, sh, dt)
    pl, y, dx, dw, db = _run_conv(sh, dt, ops)
    s, p = sh.stride, sh.padding
    ry = oracle.conv_forward(ops["x"].exact, ops["w"].exact, ops["bias"].exact, s, p)
    rdx = oracle.conv_backward_data(ops["g"].exact, ops["w"].exact, sh.x_shape(), s, p)
    rdw = oracle.conv_backward_filter(ops["x"].exact, ops["g"].exact, sh.w_shape(), s, p)
    rdb = oracle.conv_backward_bias(ops["g"].exact)
    errs = {"y": rel_err(host(y), ry), "dx": rel_err(host(dx), rdx),
            "dw": rel_err(host(dw), rdw), "db": rel_err(host(db), rdb)}
    _say("  rel errors", errs)
    for k, e in errs.items():
        assert e < TOL[dt], (tag, k, e)
    ay, adx, adw, adb = _abs_refs(sh, ops["x"].exact, ops["w"].exact, ops["g"].exact, ops["bias"].exact)
    elementwise_bound(host(y), ry, ay, sh.Kc + 1, (tag, "y"))
    elementwise_bound(host(dx), rdx, adx, sh.outC * sh.kH * sh.kW + 1, (tag, "dx"))
    elementwise_bound(host(dw), rdw, adw, sh.N, (tag, "dw"))
    elementwise_bound(host(db), rdb, adb, sh.N, (tag, "db"))
    return y, dx, dw, db


@pytest.mark.parametrize("t", TINY, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_conv_tiny_shapes(t, dt):
    sh = _shape(t)
    ops = wl.random_conv(sh, dt, seed=sum(t))
    _check_whole(sh, dt, ops, "tiny")


def _config_cases(max_batch):
    out = []
    for key, w in wl.WORKLOADS.items():
        for li, layer in enumerate(w.layers):
            for dt in w.dtypes:
                out.append((key, li, dt, min(layer.shape.batch, max_batch[key])))
    return out


REDUCED = {"c1": 8, "c2": 64, "c3": 2, "c4": 3, "c5": 1}


@pytest.mark.parametrize("key,li,dt,batch", _config_cases(REDUCED), ids=str)
def test_conv_config_whole_tensor(key, li, dt, batch):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape.with_batch(batch)
    ops = wl.conv_inputs(w, li, dt, batch=batch)
    _check_whole(sh, dt, ops, f"{key}/{w.layers[li].name}/b{batch}")


def test_c2_fc_gemms():
    w = wl.WORKLOADS["c2"]
    for i, c in enumerate(w.gemms):
        ops = wl.gemm_inputs(w, i, "f32")
        ref = oracle.gemm(ops["A"].exact, ops["B"].exact, c.M, c.K, c.N, c.flags)
        C = d4r.gemm(dev(ops["A"]), dev(ops["B"]), c.M, c.K, c.N, c.flags)
        torch.cuda.synchronize()
        err = rel_err(host(C), ref)
        _say("fc", c.name, err)
        assert err < TOL["f32"], (c.name, err)


# ---------------------------------------------------------------------------
# full-size parity on sampled blocks (the bench's launch configuration)
# ---------------------------------------------------------------------------

def _sample_idx(n, k):
    return np.unique(np.linspace(0, n - 1, num=min(n, k)).round().astype(int))


@pytest.mark.parametrize("key,li,dt", [(k, li, dt) for k, w in wl.WORKLOADS.items()
                                       for li in range(len(w.layers)) for dt in w.dtypes], ids=str)
def test_conv_full_size_sampled(key, li, dt):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape
    ops = wl.conv_inputs(w, li, dt)
    _say("full-size", key, w.layers[li].name, dt, sh)
    pl, y, dx, dw, db = _run_conv(sh, dt, ops)
    s, p = sh.stride, sh.padding
    X, Wt, G, bias = ops["x"].exact, ops["w"].exact, ops["g"].exact, ops["bias"].exact
    bs = _sample_idx(sh.batch, 2)
    os_ = _sample_idx(sh.outC, 6)
    cs = _sample_idx(sh.inC, 6)
    ry = oracle.conv_forward(X[bs], Wt[os_], bias[os_], s, p)
    gy = host(y)[np.ix_(bs, os_)]
    rdx = oracle.conv_backward_data(G[bs], Wt[:, cs], (len(bs), len(cs), sh.inH, sh.inW), s, p)
    gdx = host(dx)[np.ix_(bs, cs)]
    rdw = oracle.conv_backward_filter(X[:, cs], G[:, os_], (len(os_), len(cs), sh.kH, sh.kW), s, p)
    gdw = host(dw)[np.ix_(os_, cs)]
    rdb = oracle.conv_backward_bias(G)
    errs = {"y": rel_err(gy, ry), "dx": rel_err(gdx, rdx), "dw": rel_err(gdw, rdw),
            "db": rel_err(host(db), rdb)}
    _say("  sampled rel errors", errs)
    for k, e in errs.items():
        assert e < TOL[dt], (k, e)
    ax, aw, ag = np.abs(X), np.abs(Wt), np.abs(G)
    elementwise_bound(gy, ry, oracle.conv_forward(ax[bs], aw[os_], np.abs(bias[os_]), s, p), sh.Kc + 1, "y")
    elementwise_bound(gdx, rdx, oracle.conv_backward_data(ag[bs], aw[:, cs], (len(bs), len(cs), sh.inH, sh.inW),
                                                          s, p), sh.outC * sh.kH * sh.kW + 1, "dx")
    elementwise_bound(gdw, rdw, oracle.conv_backward_filter(ax[:, cs], ag[:, os_], (len(os_), len(cs), sh.kH, sh.kW),
                                                            s, p), sh.N, "dw")
    elementwise_bound(host(db), rdb, oracle.conv_backward_bias(ag), sh.N, "db")
    # independent of the oracle: <y - bias, g> = <x, dx> = <W, dW>
    ysb = host(y) - bias[None, :, None, None]
    lhs = float(np.vdot(ysb, G))
    scale = float(np.abs(ysb).ravel() @ np.abs(G).ravel()) + 1.0
    assert abs(lhs - float(np.vdot(X, host(dx)))) / scale < 1e-5
    assert abs(lhs - float(np.vdot(Wt, host(dw)))) / scale < 1e-5


# ---------------------------------------------------------------------------
# determinism and the saved-col contract
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bitwise_deterministic(dt):
    w = wl.WORKLOADS["c4"]
    sh = w.layers[1].shape.with_batch(8)
    ops = wl.conv_inputs(w, 1, dt, batch=8)
    a = _run_conv(sh, dt, ops)[1:]
    b = _run_conv(sh, dt, ops)[1:]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_reuse_col_matches_fresh_im2col():
    w = wl.WORKLOADS["c3"]
    sh = w.layers[0].shape.with_batch(2)
    ops = wl.conv_inputs(w, 0, "f32", batch=2)
    pl = _plan(sh, "f32")
    x, wt, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl.forward(x, wt, dev(ops["bias"]))
    pl.backward_data(wt, g)          # must not disturb the saved col
    dw1, db1 = pl.backward_filter(None, g, reuse_col=True)
    dw2, db2 = pl.backward_filter(x, g, reuse_col=False)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2) and torch.equal(db1, db2)


@pytest.mark.parametrize("path", ["inplace", "copy"])
def test_filter_gradient_without_bias(path, monkeypatch):
    # db = NULL skips the bias gradient on both ways of taking dy (the copy
    # path otherwise folds the bias partial sums into its reshape)
    monkeypatch.setenv("D4R_GRAD_PATH", path)
    sh = _shape((3, 5, 9, 9, 37, 3, 3, 1, 1))
    ops = wl.random_conv(sh, "f32", seed=5)
    pl = _plan(sh, "f32")
    pl.forward(dev(ops["x"]), dev(ops["w"]), dev(ops["bias"]))
    dw, db = pl.backward_filter(None, dev(ops["g"]), reuse_col=True, want_bias=False)
    torch.cuda.synchronize()
    assert db is None
    ref = oracle.conv_backward_filter(ops["x"].exact, ops["g"].exact, sh.w_shape(), 1, 1)
    assert rel_err(host(dw), ref) < 1e-5


def test_forward_without_bias():
    sh = _shape((2, 3, 9, 9, 4, 3, 3, 1, 1))
    ops = wl.random_conv(sh, "f32", seed=3)
    pl = _plan(sh, "f32")
    y = pl.forward(dev(ops["x"]), dev(ops["w"]), None)
    torch.cuda.synchronize()
    ref = oracle.conv_forward(ops["x"].exact, ops["w"].exact, None, 1, 1)
    assert rel_err(host(y), ref) < 1e-5


# ---------------------------------------------------------------------------
# every GEMM tile configuration on ragged shapes (planner override)
# ---------------------------------------------------------------------------

TILES = {"f32": ["128x128", "64x64", "32x128", "96x128", "128x64"],
         "f16": ["128x128", "64x64", "32x128", "96x128", "128x256", "256x128", "256x256"],
         "bf16": ["128x128", "64x64", "32x128", "96x128", "128x256", "256x128", "256x256"]}


@pytest.mark.parametrize("dt,tile", [(d, t) for d in TILES for t in TILES[d]])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_gemm_every_tile_config(dt, tile, flags, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    # K % 64 == 0 shapes take the direct-to-LDS 16-bit kernel for flags 2 on
    # the 128x256 / 256x128 tiles; (200, 4096, 304) also splits K
    for (M, K, N) in [(300, 200, 333), (97, 1000, 65), (257, 136, 520), (300, 256, 333), (129, 64, 520),
                      (296, 256, 336), (136, 64, 520), (200, 4096, 304)]:
        rng = np.random.default_rng(M + K + N + flags)
        a = wl.quantize(rng.normal(size=(K, M) if flags & 1 else (M, K)), dt)
        b = wl.quantize(rng.normal(size=(N, K) if flags & 2 else (K, N)), dt)
        ref = oracle.gemm(a.exact, b.exact, M, K, N, flags)
        C = d4r.gemm(dev(a), dev(b), M, K, N, flags)
        torch.cuda.synchronize()
        err = rel_err(host(C), ref)
        assert err < TOL[dt], (tile, M, K, N, err)


# The direct-to-LDS kernel takes two k-contiguous operands (flags 2) on the
# f32 128x128 / 128x64 and 16-bit 128x128 tiles by default; the switches
# below run the register-staged kernels those GEMMs would otherwise use.
@pytest.mark.parametrize("dt,tile,switch", [("f32", "128x128", "D4R_F32_DL"), ("f32", "128x64", "D4R_F32_DL"),
                                            ("f16", "128x128", "D4R_DL128"), ("bf16", "128x128", "D4R_DL128")])
@pytest.mark.parametrize("direct", [True, False])
def test_gemm_direct_and_register_staged(dt, tile, switch, direct, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    monkeypatch.setenv(switch, "1" if direct else "0")
    for (M, K, N) in [(300, 256, 333), (129, 64, 520), (296, 256, 336), (200, 4096, 304), (70, 96, 36)]:
        rng = np.random.default_rng(M + K + N + 7)
        a = wl.quantize(rng.normal(size=(M, K)), dt)
        b = wl.quantize(rng.normal(size=(N, K)), dt)
        ref = oracle.gemm(a.exact, b.exact, M, K, N, 2)
        C = d4r.gemm(dev(a), dev(b), M, K, N, 2)
        torch.cuda.synchronize()
        err = rel_err(host(C), ref)
        assert err < TOL[dt], (tile, direct, M, K, N, err)


# The 16-bit direct-to-LDS 128x128 tile in each of its forms (four
# wavefronts of 64x64 or eight of 64x32; rings of two to four stages) on the
# ragged direct-kernel GEMM shapes and on a conv3-5 layer.
@pytest.mark.parametrize("form", ["w4n2", "w8n2", "w8n3", "w8n4"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_dl128_forms(form, dt, monkeypatch):
    monkeypatch.setenv("D4R_DL128_FORM", form)
    monkeypatch.setenv("D4R_GEMM_TILE", "128x128")
    for (M, K, N) in [(300, 256, 333), (129, 64, 520), (200, 4096, 304), (70, 128, 36)]:
        rng = np.random.default_rng(M + K + N + 13)
        a = wl.quantize(rng.normal(size=(M, K)), dt)
        b = wl.quantize(rng.normal(size=(N, K)), dt)
        ref = oracle.gemm(a.exact, b.exact, M, K, N, 2)
        C = d4r.gemm(dev(a), dev(b), M, K, N, 2)
        torch.cuda.synchronize()
        err = rel_err(host(C), ref)
        assert err < TOL[dt], (form, M, K, N, err)
    w = wl.WORKLOADS["c4"]
    sh = w.layers[1].shape.with_batch(3)
    _check_whole(sh, dt, wl.conv_inputs(w, 1, dt, batch=3), f"c4/conv4/b3/{form}")


# The 16-bit direct-to-LDS kernels' two loops (fragment reads pipelined one
# k step ahead, the default; the plain loop with D4R_DL16_PIPE=0) on every
# direct tile over ragged shapes (one stage, split K, rows and columns past
# the matrix), on a conv3-5 layer (NHWC forward and data gradient, filter
# gradient) and on the phased data gradient of strided layers.
@pytest.mark.parametrize("pipe", ["1", "0"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_dl16_loop_forms(pipe, dt, monkeypatch):
    monkeypatch.setenv("D4R_DL16_PIPE", pipe)
    for tile in ["128x128", "128x256", "256x128", "256x256"]:
        monkeypatch.setenv("D4R_GEMM_TILE", tile)
        for (M, K, N) in [(300, 256, 333), (129, 64, 520), (200, 4096, 304), (513, 640, 257)]:
            rng = np.random.default_rng(M + K + N + 41)
            a = wl.quantize(rng.normal(size=(M, K)), dt)
            b = wl.quantize(rng.normal(size=(N, K)), dt)
            ref = oracle.gemm(a.exact, b.exact, M, K, N, 2)
            C = d4r.gemm(dev(a), dev(b), M, K, N, 2)
            torch.cuda.synchronize()
            got = host(C)
            assert rel_err(got, ref) < TOL[dt], (pipe, tile, M, K, N)
            elementwise_bound(got, ref, oracle.gemm(np.abs(a.exact), np.abs(b.exact), M, K, N, 2), K,
                              f"C pipe={pipe} {tile} {M}x{K}x{N}")
    monkeypatch.delenv("D4R_GEMM_TILE")
    w = wl.WORKLOADS["c4"]
    sh = w.layers[2].shape.with_batch(3)
    _check_whole(sh, dt, wl.conv_inputs(w, 2, dt, batch=3), f"c4/conv5/b3/pipe{pipe}")
    for t in [(2, 64, 9, 11, 64, 3, 3, 2, 1), (1, 64, 12, 12, 64, 11, 11, 4, 2)]:
        shp = _shape(t)
        _check_dgrad_implicit(shp, dt, wl.random_conv(shp, dt, seed=sum(t) + 43), f"phased pipe={pipe}")


# large k-contiguous products: the 256x256 tile, and grids of 16+ tiles each
# way, which run in bands of 8 M tiles (ragged last band and tiles)
@pytest.mark.parametrize("dt,M,K,N", [("f16", 2048, 2048, 2048), ("bf16", 2048, 2048, 2048),
                                      ("bf16", 4000, 128, 4100), ("f16", 4200, 192, 3900),
                                      ("f32", 2100, 96, 2050)])
def test_gemm_large_sampled(dt, M, K, N):
    rng = np.random.default_rng(M + K + N)
    a = wl.quantize(rng.normal(size=(M, K)), dt)
    b = wl.quantize(rng.normal(size=(N, K)), dt)
    C = d4r.gemm(dev(a), dev(b), M, K, N, 2)
    torch.cuda.synchronize()
    rows = _sample_idx(M, 40)
    ref = oracle.gemm(a.exact[rows].copy(), b.exact, len(rows), K, N, 2)
    got = host(C)[rows]
    assert rel_err(got, ref) < TOL[dt]
    elementwise_bound(got, ref, oracle.gemm(np.abs(a.exact[rows]), np.abs(b.exact), len(rows), K, N, 2), K,
                      "C")


@pytest.mark.parametrize("dt,switch", [("f32", "D4R_F32_DL"), ("bf16", "D4R_DL128")])
def test_conv_c4_register_staged_gradients(dt, switch, monkeypatch):
    # conv5 at batch 3 with the direct-to-LDS kernel switched off: the
    # register-staged filter-gradient GEMM and NHWC data gradient
    monkeypatch.setenv(switch, "0")
    w = wl.WORKLOADS["c4"]
    sh = w.layers[2].shape.with_batch(3)
    _check_whole(sh, dt, wl.conv_inputs(w, 2, dt, batch=3), f"c4/conv5/b3/{switch}=0")


# f32 conv passes with every tile and both ways of taking dy in the gradient
# GEMMs (read in place by the NCHW operand loaders, or copied first), over
# odd pixel counts whose images straddle tiles, with and without 16-byte
# vector loads on the other operand (Kc % 4).
CONV_TILE_SHAPES = [
    (5, 5, 9, 9, 37, 3, 3, 1, 1),     # P = 81, Kc = 45, N = 405
    (7, 8, 13, 13, 40, 3, 3, 2, 1),   # P = 49, Kc = 72, N = 343
    (3, 4, 11, 10, 130, 1, 1, 1, 0),  # P = 110, Kc = 4, O > 128
]


@pytest.mark.parametrize("path", ["inplace", "copy"])
@pytest.mark.parametrize("tile", TILES["f32"])
@pytest.mark.parametrize("t", CONV_TILE_SHAPES, ids=str)
def test_conv_f32_every_tile(tile, t, path, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    monkeypatch.setenv("D4R_GRAD_PATH", path)
    sh = _shape(t)
    _check_whole(sh, "f32", wl.random_conv(sh, "f32", seed=sum(t) + 3), f"tile {tile}")


@pytest.mark.parametrize("li", [0, 1, 2])
def test_conv_c4_f32_gradients_in_place(li, monkeypatch):
    # conv3-5 take the copy path by default; force the in-place loaders
    monkeypatch.setenv("D4R_GRAD_PATH", "inplace")
    w = wl.WORKLOADS["c4"]
    sh = w.layers[li].shape.with_batch(3)
    _check_whole(sh, "f32", wl.conv_inputs(w, li, "f32", batch=3), f"c4/{w.layers[li].name}/b3/inplace")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_conv_data_gradient_w_row_contiguous(dt, monkeypatch):
    # the copy path transposes W for the data gradient by default; force the
    # GEMM that reads W row-contiguous instead
    monkeypatch.setenv("D4R_DGRAD_WT", "0")
    w = wl.WORKLOADS["c4"]
    sh = w.layers[2].shape.with_batch(3)
    _check_whole(sh, dt, wl.conv_inputs(w, 2, dt, batch=3), f"c4/conv5/b3/w-rows")


@pytest.mark.parametrize("tile", ["128x128", "128x256", "256x128"])
def test_conv_bf16_every_big_tile(tile, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    w = wl.WORKLOADS["c4"]
    sh = w.layers[2].shape.with_batch(3)
    ops = wl.conv_inputs(w, 2, "bf16", batch=3)
    _check_whole(sh, "bf16", ops, f"c4/conv5/b3/{tile}")


# ---------------------------------------------------------------------------
# implicit-GEMM forward (no col matrix in HBM)
# ---------------------------------------------------------------------------

def _check_implicit(sh, dt, ops, tag, sample=False):
    _say("implicit fwd", tag, sh, dt)
    pl = _plan(sh, dt)
    x, w, bias = dev(ops["x"]), dev(ops["w"]), dev(ops["bias"])
    y = pl.forward_implicit(x, w, bias)
    y2 = pl.forward(x, w, bias)
    torch.cuda.synchronize()
    s, p = sh.stride, sh.padding
    if sample:
        bs = _sample_idx(sh.batch, 2)
        os_ = _sample_idx(sh.outC, 6)
        ref = oracle.conv_forward(ops["x"].exact[bs], ops["w"].exact[os_], ops["bias"].exact[os_], s, p)
        got = host(y)[np.ix_(bs, os_)]
    else:
        ref = oracle.conv_forward(ops["x"].exact, ops["w"].exact, ops["bias"].exact, s, p)
        got = host(y)
    err = rel_err(got, ref)
    _say("  rel err", err, "vs explicit", rel_err(host(y), host(y2)))
    assert err < TOL[dt], (tag, err)


@pytest.mark.parametrize("t", TINY, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_implicit_forward_tiny(t, dt):
    sh = _shape(t)
    _check_implicit(sh, dt, wl.random_conv(sh, dt, seed=sum(t) + 7), "tiny")


@pytest.mark.parametrize("key,li,dt,batch", _config_cases(REDUCED), ids=str)
def test_implicit_forward_configs(key, li, dt, batch):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape.with_batch(batch)
    _check_implicit(sh, dt, wl.conv_inputs(w, li, dt, batch=batch), f"{key}/{w.layers[li].name}/b{batch}")


@pytest.mark.parametrize("key,li,dt", [(k, li, dt) for k, w in wl.WORKLOADS.items()
                                       for li in range(len(w.layers)) for dt in w.dtypes], ids=str)
def test_implicit_forward_full_size_sampled(key, li, dt):
    w = wl.WORKLOADS[key]
    _check_implicit(w.layers[li].shape, dt, wl.conv_inputs(w, li, dt), f"{key}/full", sample=True)


@pytest.mark.parametrize("dt,tile", [(d, t) for d in TILES for t in TILES[d]])
def test_implicit_forward_every_tile(dt, tile, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    sh = _shape((3, 7, 23, 29, 65, 5, 3, 2, 2))
    _check_implicit(sh, dt, wl.random_conv(sh, dt, seed=11), f"tile {tile}")
    sh = _shape((2, 17, 12, 12, 130, 3, 3, 1, 1))
    _check_implicit(sh, dt, wl.random_conv(sh, dt, seed=12), f"tile {tile}")


# implicit forward from x read as NHWC (input channels a multiple of the
# GEMM stage: 32 f32, 64 16-bit; the 16-bit one on the direct-to-LDS
# kernel): ragged pixel counts and output channels, padding above kH - 1,
# non-square kernels, split K; the gathered implicit forward must agree
FWD_NHWC = [
    (2, 64, 8, 7, 5, 3, 3, 1, 1),
    (3, 128, 9, 11, 40, 3, 3, 1, 0),
    (2, 64, 7, 7, 130, 3, 3, 1, 2),
    (1, 192, 6, 6, 16, 5, 5, 1, 2),
    (2, 64, 5, 5, 8, 3, 3, 1, 3),
    (2, 64, 6, 9, 33, 2, 3, 1, 1),
    (4, 256, 5, 9, 24, 3, 3, 1, 1),
    (2, 32, 5, 9, 24, 3, 3, 1, 1),
]


@pytest.mark.parametrize("t", FWD_NHWC, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_forward_implicit_nhwc(t, dt, monkeypatch):
    sh = _shape(t)
    pl = _plan(sh, dt)
    applies = sh.inC % (32 if dt == "f32" else 64) == 0
    assert d4r.d4r_conv_describe(pl.h)["fwd_implicit"] == ("nhwc" if applies else "gathered")
    ops = wl.random_conv(sh, dt, seed=sum(t) + 29)
    _check_implicit(sh, dt, ops, "nhwc")
    monkeypatch.setenv("D4R_FWD_NHWC", "0")
    _check_implicit(sh, dt, ops, "gathered")


# ---------------------------------------------------------------------------
# implicit-GEMM data gradient (stride 1, square kernel: no dcol, no col2im;
# other shapes take the explicit path through the same entry point)
# ---------------------------------------------------------------------------

def _check_dgrad_implicit(sh, dt, ops, tag, sample=False):
    _say("implicit dgrad", tag, sh, dt)
    pl = _plan(sh, dt)
    w, g = dev(ops["w"]), dev(ops["g"])
    dx = pl.backward_data_implicit(w, g)
    dx2 = pl.backward_data(w, g)
    torch.cuda.synchronize()
    s, p = sh.stride, sh.padding
    if sample:
        bs = _sample_idx(sh.batch, 2)
        cs = _sample_idx(sh.inC, 6)
        ref = oracle.conv_backward_data(ops["g"].exact[bs], ops["w"].exact[:, cs],
                                        (len(bs), len(cs), sh.inH, sh.inW), s, p)
        got = host(dx)[np.ix_(bs, cs)]
    else:
        ref = oracle.conv_backward_data(ops["g"].exact, ops["w"].exact, sh.x_shape(), s, p)
        got = host(dx)
    err = rel_err(got, ref)
    _say("  rel err", err, "vs explicit", rel_err(host(dx), host(dx2)))
    assert err < TOL[dt], (tag, err)


# stride 1 with padding below, at and above kH - 1 (negative flipped padding)
DGRAD_TINY = TINY + [
    (2, 3, 8, 7, 4, 3, 3, 1, 0),
    (2, 3, 8, 7, 4, 3, 3, 1, 2),
    (1, 2, 6, 6, 3, 2, 2, 1, 3),
    (2, 4, 9, 11, 5, 5, 5, 1, 2),
    (3, 5, 7, 7, 6, 1, 1, 1, 0),
    # dy channels a multiple of the GEMM stage and padding above kH - 1: the
    # NHWC path with a negative flipped padding (kH - 1 - p < 0)
    (2, 32, 6, 6, 64, 2, 2, 1, 3),
    (1, 64, 5, 5, 128, 3, 3, 1, 3),
]


@pytest.mark.parametrize("t", DGRAD_TINY, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_implicit_dgrad_tiny(t, dt):
    sh = _shape(t)
    _check_dgrad_implicit(sh, dt, wl.random_conv(sh, dt, seed=sum(t) + 17), "tiny")


@pytest.mark.parametrize("key,li,dt,batch", _config_cases(REDUCED), ids=str)
def test_implicit_dgrad_configs(key, li, dt, batch):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape.with_batch(batch)
    _check_dgrad_implicit(sh, dt, wl.conv_inputs(w, li, dt, batch=batch), f"{key}/{w.layers[li].name}/b{batch}")


@pytest.mark.parametrize("key,li,dt", [(k, li, dt) for k, w in wl.WORKLOADS.items() if k in ("c4", "c5")
                                       for li in range(len(w.layers)) for dt in w.dtypes], ids=str)
def test_implicit_dgrad_full_size_sampled(key, li, dt):
    w = wl.WORKLOADS[key]
    _check_dgrad_implicit(w.layers[li].shape, dt, wl.conv_inputs(w, li, dt), f"{key}/full", sample=True)


@pytest.mark.parametrize("dt,tile", [(d, t) for d in TILES for t in TILES[d]])
def test_implicit_dgrad_every_tile(dt, tile, monkeypatch):
    monkeypatch.setenv("D4R_GEMM_TILE", tile)
    sh = _shape((3, 37, 9, 10, 21, 3, 3, 1, 1))
    _check_dgrad_implicit(sh, dt, wl.random_conv(sh, dt, seed=23), f"tile {tile}")


def test_implicit_dgrad_keeps_saved_col():
    w = wl.WORKLOADS["c4"]
    sh = w.layers[0].shape.with_batch(2)
    ops = wl.conv_inputs(w, 0, "f32", batch=2)
    pl = _plan(sh, "f32")
    x, wt, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
    pl.forward(x, wt, dev(ops["bias"]))
    pl.backward_data_implicit(wt, g)   # must not disturb the saved col
    dw1, db1 = pl.backward_filter(None, g, reuse_col=True)
    dw2, db2 = pl.backward_filter(x, g, reuse_col=False)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2) and torch.equal(db1, db2)


# implicit data gradient from dy read as NHWC (dy channels a multiple of the
# GEMM stage: 32 f32, 64 16-bit, the latter through the direct-to-LDS
# kernel): padding below, at and above kH - 1, pixel counts that leave
# ragged tiles, input channels that do not fill a tile row, and split K
DGRAD_NHWC = [
    (2, 3, 8, 7, 64, 3, 3, 1, 1),
    (3, 40, 9, 11, 128, 3, 3, 1, 0),
    (2, 130, 7, 7, 64, 3, 3, 1, 2),
    (1, 16, 6, 6, 192, 5, 5, 1, 2),
    (2, 8, 13, 13, 64, 3, 3, 1, 3),
    (4, 24, 5, 9, 256, 3, 3, 1, 1),
]


@pytest.mark.parametrize("t", DGRAD_NHWC, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_dgrad_implicit_nhwc(t, dt, monkeypatch):
    sh = _shape(t)
    ops = wl.random_conv(sh, dt, seed=sum(t) + 21)
    _check_dgrad_implicit(sh, dt, ops, "nhwc")
    # the gathered implicit path agrees
    monkeypatch.setenv("D4R_DGRAD_NHWC", "0")
    _check_dgrad_implicit(sh, dt, ops, "gathered")


# strided layers: stride^2 stride-1 sub-convolutions of dy (one per output
# phase) in one launch, no dcol, no col2im; stride 2 to 4, ragged input
# channel counts, non-square kernels, per-axis and negative paddings
DGRAD_PHASED = [
    (2, 64, 9, 11, 64, 3, 3, 2, 1),
    (1, 96, 10, 9, 128, 5, 5, 2, 2),
    (2, 64, 13, 12, 64, 4, 4, 3, 1),
    (1, 64, 12, 12, 64, 11, 11, 4, 2),
    (2, 130, 7, 8, 64, 3, 2, 2, 0),
    (1, 64, 8, 10, 64, 3, 3, 3, 3),
    (3, 64, 6, 5, 192, 2, 2, 2, 1),
]


@pytest.mark.parametrize("t", DGRAD_PHASED, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_dgrad_phased(t, dt, monkeypatch):
    sh = _shape(t)
    pl = _plan(sh, dt)      # keeps the handle alive while it is described
    assert d4r.d4r_conv_describe(pl.h)["dgrad_implicit"] == "phased"
    ops = wl.random_conv(sh, dt, seed=sum(t) + 37)
    _check_dgrad_implicit(sh, dt, ops, "phased")
    monkeypatch.setenv("D4R_DGRAD_PHASED", "0")
    pl = _plan(sh, dt)
    assert d4r.d4r_conv_describe(pl.h)["dgrad_implicit"] == "explicit"
    _check_dgrad_implicit(sh, dt, ops, "explicit")


# Layers with few input channels, where the planner keeps the explicit data
# gradient (its GEMM rows are C*kH*kW) and D4R_DGRAD_PHASED=force takes the
# phased one: AlexNet conv1's geometry (3 channels, 11x11, stride 4) at
# batch 2, and small ragged cases (f32: dy channels a multiple of 32)
DGRAD_PHASED_FORCED = [
    (2, 3, 224, 224, 96, 11, 11, 4, 2),
    (2, 3, 23, 21, 32, 5, 5, 2, 1),
    (1, 5, 17, 19, 64, 7, 5, 3, 2),
]


@pytest.mark.parametrize("t", DGRAD_PHASED_FORCED, ids=str)
def test_dgrad_phased_forced_few_channels(t, monkeypatch):
    sh = _shape(t)
    pl = _plan(sh, "f32")
    assert d4r.d4r_conv_describe(pl.h)["dgrad_implicit"] == "explicit"
    monkeypatch.setenv("D4R_DGRAD_PHASED", "force")
    pl = _plan(sh, "f32")
    d = d4r.d4r_conv_describe(pl.h)
    assert d["dgrad_implicit"] == "phased" and int(d["dgrad_phases"]) == sh.stride ** 2, d
    ops = wl.random_conv(sh, "f32", seed=sum(t) + 41)
    _check_dgrad_implicit(sh, "f32", ops, "phased (forced)")


def test_dgrad_phased_applies_to_the_workloads():
    # the 46x80 map's stride-2 layer takes it; AlexNet conv1 (3 input channels) does not
    c5 = wl.WORKLOADS["c5"].layers[2].shape
    c3 = wl.WORKLOADS["c3"].layers[0].shape
    p5, p3 = _plan(c5, "f16"), _plan(c3, "f32")
    d5 = d4r.d4r_conv_describe(p5.h)
    assert d5["dgrad_implicit"] == "phased" and d5["dgrad_phases"] == "4"
    assert d4r.d4r_conv_describe(p3.h)["dgrad_implicit"] == "explicit"


@pytest.mark.parametrize("key,li,dt", [("c4", 0, "bf16"), ("c4", 1, "bf16"), ("c4", 2, "bf16"), ("c5", 0, "f16"),
                                       ("c4", 1, "f32"), ("c5", 2, "f16")])
def test_dgrad_implicit_nhwc_full_size(key, li, dt):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape
    ops = wl.conv_inputs(w, li, dt)
    _check_dgrad_implicit(sh, dt, ops, f"{key}/{w.layers[li].name}/nhwc", sample=True)
