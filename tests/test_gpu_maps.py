"""GPU parity of the index maps in the bench's launch configuration, of the
standalone bias gradient, and guard bands around every output.

* im2col and col2im bit-exact against the oracle's index-map specifications
  at the full batch of every workload layer, where the launchers pick
  multi-image LDS windows (asserted through d4r_conv_describe), and with the
  shifted-copy im2col switched off so the general LDS kernel runs too.
  im2col: float32 iota codes (exact below 2^24) and raw 16-bit patterns;
  col2im: small-integer dcol, whose sums are exact in float32.
* d4r_conv_bias_grad against the oracle's per-channel sum.
* Guard bands: every output (y, dx, dw, db, col, C, the workspace) is an
  interior view of a larger buffer filled with a NaN sentinel; after the
  call every sentinel word must be unchanged, so no kernel stores past
  either end of its output on ragged shapes.
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

SENTINEL = 0x7FBADBAD          # a quiet-NaN pattern no kernel writes
PAD_WORDS = 68                 # 272 bytes: 16-byte aligned, not 256-byte aligned


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


def _plan(sh, dt):
    return d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding,
                        sh.outC, DT_CODE[dt])


def _layers():
    for key, w in wl.WORKLOADS.items():
        for li, layer in enumerate(w.layers):
            yield key, li, layer


# ---------------------------------------------------------------------------
# full-batch index maps
# ---------------------------------------------------------------------------

def _im2col_full_cases():
    out = []
    for key, li, layer in _layers():
        for dt in wl.WORKLOADS[key].dtypes:
            out.append((key, li, dt, "1"))
            sh = layer.shape
            if sh.stride == 1:
                out.append((key, li, dt, "0"))   # general LDS kernel instead of shifted copies
    return out


def _im2col_check(sh, dt):
    n = int(np.prod(sh.x_shape()))
    codes = np.arange(1, n + 1, dtype=np.int64)
    if dt == "f32":
        assert n < 2 ** 24
        x = torch.from_numpy(codes.astype(np.float32).reshape(sh.x_shape())).cuda()
        src = codes
    else:
        src = (codes * 2654435761) % 65521 + 1          # nonzero 16-bit patterns
        x = torch.from_numpy(src.astype(np.uint16).view(np.int16).reshape(sh.x_shape())).cuda()
        x = x.view(torch.bfloat16 if dt == "bf16" else torch.float16)
    ref = oracle.im2col_spec(src.reshape(sh.x_shape()).astype(np.float64), sh.kH, sh.kW, sh.stride,
                             sh.padding)
    pl = _plan(sh, dt)
    col = torch.empty((sh.Kc, sh.N), dtype=x.dtype, device="cuda")
    d4r.d4r_conv_im2col(pl.h, x, col)
    torch.cuda.synchronize()
    if dt == "f32":
        got = col.cpu().numpy().astype(np.float64)
    else:
        got = bits16(col).astype(np.float64)
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{bad} of {ref.size} col entries differ"
    return pl


@pytest.mark.parametrize("key,li,dt,shift", _im2col_full_cases(), ids=str)
def test_im2col_bit_exact_full_batch(key, li, dt, shift, monkeypatch):
    monkeypatch.setenv("D4R_IM2COL_SHIFT", shift)
    sh = wl.WORKLOADS[key].layers[li].shape
    pl = _plan(sh, dt)
    plan = d4r.d4r_conv_describe(pl.h)
    _say("im2col full", key, li, dt, sh, {k: plan[k] for k in ("im2col", "im2col_rb", "im2col_bb")})
    if shift == "0":
        assert plan["im2col"] != "shift"
    # AlexNet conv3-5 (13x13 planes, batch 64): several images per block at
    # full size, the launch configuration the bench times (the other layers
    # need one image or a row range per block to fill the chip)
    if key == "c4":
        assert plan["im2col"] != "gather" and int(plan["im2col_bb"]) > 1, plan
    _im2col_check(sh, dt)


@pytest.mark.parametrize("key,li", [(k, li) for k, li, _ in _layers()], ids=str)
def test_col2im_bit_exact_full_batch(key, li):
    sh = wl.WORKLOADS[key].layers[li].shape
    pl = _plan(sh, "f32")
    plan = d4r.d4r_conv_describe(pl.h)
    _say("col2im full", key, li, sh, {k: plan[k] for k in ("col2im", "col2im_bb")})
    if key == "c4":
        assert plan["col2im"] == "lds" and int(plan["col2im_bb"]) > 1, plan
    rng = np.random.default_rng(1000 + 10 * li + wl.WORKLOADS[key].cfg_id)
    dcol = rng.integers(-8, 9, size=(sh.Kc, sh.N)).astype(np.float32)
    ref = oracle.col2im_spec(dcol.astype(np.float64), sh.x_shape(), sh.kH, sh.kW, sh.stride, sh.padding)
    dx = torch.empty(sh.x_shape(), dtype=torch.float32, device="cuda")
    d4r.d4r_conv_col2im(pl.h, torch.from_numpy(dcol).cuda(), dx)
    torch.cuda.synchronize()
    got = dx.cpu().numpy().astype(np.float64)
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{bad} of {ref.size} dx entries differ"


# Multi-image col2im windows on shapes with ragged image groups (B not a
# multiple of the images per block) and every stride the LDS kernel takes.
COL2IM_MULTI = [(37, 256, 9, 9, 3, 3, 3, 1, 1), (29, 128, 12, 11, 2, 5, 3, 2, 2), (33, 64, 15, 13, 4, 3, 3, 3, 0),
                (41, 96, 8, 8, 2, 2, 2, 2, 0)]


@pytest.mark.parametrize("t", COL2IM_MULTI, ids=str)
def test_col2im_multi_image_windows(t, monkeypatch):
    B, C, H, W, O, kH, kW, s, p = t
    sh = wl.ConvShape(B, C, H, W, kH, kW, s, p, O)
    pl = _plan(sh, "f32")
    plan = d4r.d4r_conv_describe(pl.h)
    _say("col2im multi", sh, plan["col2im"], plan["col2im_bb"])
    bb = int(plan["col2im_bb"])
    assert plan["col2im"] == "lds" and bb > 1 and B % bb != 0, plan
    rng = np.random.default_rng(sum(t))
    dcol = rng.integers(-8, 9, size=(sh.Kc, sh.N)).astype(np.float32)
    ref = oracle.col2im_spec(dcol.astype(np.float64), sh.x_shape(), kH, kW, s, p)
    dx = torch.empty(sh.x_shape(), dtype=torch.float32, device="cuda")
    d4r.d4r_conv_col2im(pl.h, torch.from_numpy(dcol).cuda(), dx)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy().astype(np.float64), ref)


# ---------------------------------------------------------------------------
# standalone bias gradient
# ---------------------------------------------------------------------------

BIAS_TINY = [(1, 1, 5, 5, 1, 3, 3, 1, 0), (2, 3, 7, 6, 5, 3, 2, 1, 1), (3, 1, 7, 5, 2, 1, 1, 4, 0),
             (2, 17, 12, 12, 130, 3, 3, 1, 1), (5, 4, 9, 9, 37, 3, 3, 1, 1)]


def _bias_case(sh, dt, ops, tag):
    pl = _plan(sh, dt)
    db = torch.empty((sh.outC,), dtype=torch.float32, device="cuda")
    d4r.d4r_conv_bias_grad(pl.h, dev(ops["g"]), db, pl.ws, pl.ws_bytes)
    torch.cuda.synchronize()
    ref = oracle.conv_backward_bias(ops["g"].exact)
    aref = oracle.conv_backward_bias(np.abs(ops["g"].exact))
    got = host(db)
    err = rel_err(got, ref)
    _say("bias grad", tag, sh, dt, err)
    assert err < TOL[dt], err
    # per channel: float32 summation of N terms
    n = sh.N
    assert np.all(np.abs(got - ref) <= 2.0 * (n + 2) * 2.0 ** -24 * aref + 1e-30)


@pytest.mark.parametrize("t", BIAS_TINY, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_bias_grad_tiny(t, dt):
    B, C, H, W, O, kH, kW, s, p = t
    sh = wl.ConvShape(B, C, H, W, kH, kW, s, p, O)
    _bias_case(sh, dt, wl.random_conv(sh, dt, seed=sum(t) + 41), "tiny")


@pytest.mark.parametrize("key,li,dt", [(k, li, dt) for k, li, _ in _layers() for dt in wl.WORKLOADS[k].dtypes],
                         ids=str)
def test_bias_grad_full_size(key, li, dt):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape
    _bias_case(sh, dt, wl.conv_inputs(w, li, dt), f"{key}/{w.layers[li].name}")


# ---------------------------------------------------------------------------
# guard bands around outputs and the workspace
# ---------------------------------------------------------------------------

class Guarded:
    """A device buffer of `nbytes` with PAD_WORDS-word (or `pad`-byte)
    sentinel bands before and after; `.t` is the interior view."""

    def __init__(self, shape, dtype=torch.float32, pad_bytes=PAD_WORDS * 4):
        es = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if shape else 1
        body = n * es
        self.pad = pad_bytes
        total = pad_bytes + body + pad_bytes
        words = (total + 3) // 4 + 64
        self.raw = torch.full((words,), SENTINEL, dtype=torch.int32, device="cuda")
        base = self.raw.data_ptr()
        # the raw buffer is 256-byte aligned (torch's allocator); the interior
        # starts pad_bytes in
        assert base % 256 == 0
        self.body = body
        self.t = self.raw.view(torch.uint8)[pad_bytes:pad_bytes + body].view(dtype).view(shape)

    def intact(self) -> bool:
        r = self.raw.view(torch.uint8)
        lo = r[:self.pad].view(torch.int32)
        hi_start = self.pad + self.body
        hi_len = (r.numel() - hi_start) // 4 * 4
        hi_bytes = r[hi_start:hi_start + hi_len]
        # the band after the body may start at a 2-byte offset (16-bit bodies)
        ok_lo = bool(torch.all(lo == SENTINEL))
        sentinel_bytes = torch.tensor(list(SENTINEL.to_bytes(4, "little")), dtype=torch.uint8, device="cuda")
        phase = hi_start % 4
        expect = sentinel_bytes.roll(-phase).repeat(hi_len // 4)
        ok_hi = bool(torch.equal(hi_bytes, expect))
        return ok_lo and ok_hi


GUARD_SHAPES = [(3, 5, 9, 9, 37, 3, 3, 1, 1), (2, 3, 7, 6, 5, 3, 2, 1, 1), (3, 7, 23, 29, 65, 5, 3, 2, 2),
                (2, 130, 7, 7, 64, 3, 3, 1, 2), (3, 4, 11, 10, 130, 1, 1, 1, 0), (2, 40, 9, 11, 128, 3, 3, 1, 0),
                (2, 130, 9, 11, 64, 3, 3, 2, 1), (2, 64, 7, 8, 64, 3, 3, 1, 1)]


def _guarded_inputs(sh, dt, seed):
    ops = wl.random_conv(sh, dt, seed=seed)
    return ops, dev(ops["x"]), dev(ops["w"]), dev(ops["g"]), dev(ops["bias"])


@pytest.mark.parametrize("t", GUARD_SHAPES, ids=str)
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_guard_bands_conv(t, dt):
    B, C, H, W, O, kH, kW, s, p = t
    sh = wl.ConvShape(B, C, H, W, kH, kW, s, p, O)
    ops, x, w, g, bias = _guarded_inputs(sh, dt, sum(t) + 61)
    h = d4r.d4r_conv_create(B, C, H, W, kH, kW, s, p, O, DT_CODE[dt])
    try:
        wsb = d4r.d4r_conv_workspace_size(h)
        ws = Guarded((wsb,), torch.uint8, pad_bytes=256)
        y, dx, dx2, dx3, dw, db = (Guarded(sh.y_shape()), Guarded(sh.x_shape()), Guarded(sh.x_shape()),
                                   Guarded(sh.x_shape()), Guarded(sh.w_shape()), Guarded((O,)))
        dw2, db2 = Guarded(sh.w_shape()), Guarded((O,))
        col = Guarded((sh.Kc, sh.N), x.dtype)
        dbs = Guarded((O,))
        _say("guard", sh, dt)
        d4r.d4r_conv_forward(h, x, w, bias, y.t, ws.t, wsb)
        d4r.d4r_conv_backward_data(h, w, g, dx.t, ws.t, wsb)
        d4r.d4r_conv_backward_data_implicit(h, w, g, dx2.t, ws.t, wsb)
        d4r.d4r_conv_backward_filter(h, None, g, dw.t, db.t, 1, ws.t, wsb)
        d4r.d4r_conv_backward(h, x, w, g, dx3.t, dw2.t, db2.t, 0, ws.t, wsb)
        d4r.d4r_conv_im2col(h, x, col.t)
        d4r.d4r_conv_bias_grad(h, g, dbs.t, ws.t, wsb)
        torch.cuda.synchronize()
        for name, buf in (("ws", ws), ("y", y), ("dx", dx), ("dx_implicit", dx2), ("dx_combined", dx3),
                          ("dw", dw), ("db", db), ("dw_combined", dw2), ("db_combined", db2), ("col", col),
                          ("db_standalone", dbs)):
            assert buf.intact(), f"{name}: a store landed outside the output"
        # and the interiors are the right results
        ref_y = oracle.conv_forward(ops["x"].exact, ops["w"].exact, ops["bias"].exact, s, p)
        ref_dx = oracle.conv_backward_data(ops["g"].exact, ops["w"].exact, sh.x_shape(), s, p)
        ref_dw = oracle.conv_backward_filter(ops["x"].exact, ops["g"].exact, sh.w_shape(), s, p)
        ref_db = oracle.conv_backward_bias(ops["g"].exact)
        for got, ref in ((y, ref_y), (dx, ref_dx), (dx2, ref_dx), (dx3, ref_dx), (dw, ref_dw), (dw2, ref_dw),
                         (db, ref_db), (db2, ref_db), (dbs, ref_db)):
            assert rel_err(host(got.t), ref) < TOL[dt]
    finally:
        d4r.d4r_conv_destroy(h)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_guard_bands_gemm(dt, flags):
    # ragged M and N (tiles cut at both ends), K with and without split-K
    for (M, K, N) in [(97, 200, 333), (300, 256, 65), (129, 4096, 130), (7, 17, 5)]:
        rng = np.random.default_rng(M + K + N + flags + 71)
        a = wl.quantize(rng.normal(size=(K, M) if flags & 1 else (M, K)), dt)
        b = wl.quantize(rng.normal(size=(N, K) if flags & 2 else (K, N)), dt)
        C = Guarded((M, N))
        wsb = d4r.d4r_gemm_workspace_size(M, K, N, flags, DT_CODE[dt])
        ws = Guarded((max(wsb, 1),), torch.uint8, pad_bytes=256)
        d4r.d4r_gemm(M, K, N, flags, DT_CODE[dt], dev(a), dev(b), C.t, ws.t if wsb else None, wsb)
        torch.cuda.synchronize()
        assert C.intact() and ws.intact(), (M, K, N, flags)
        ref = oracle.gemm(a.exact, b.exact, M, K, N, flags)
        assert rel_err(host(C.t), ref) < TOL[dt]


def test_guard_bands_col2im():
    sh = wl.ConvShape(3, 5, 9, 9, 3, 3, 1, 1, 4)
    pl = _plan(sh, "f32")
    dcol = torch.ones((sh.Kc, sh.N), dtype=torch.float32, device="cuda")
    dx = Guarded(sh.x_shape())
    d4r.d4r_conv_col2im(pl.h, dcol, dx.t)
    sh2 = wl.ConvShape(2, 3, 30, 30, 11, 11, 4, 2, 4)    # element-parallel gather
    pl2 = _plan(sh2, "f32")
    dx2 = Guarded(sh2.x_shape())
    d4r.d4r_conv_col2im(pl2.h, torch.ones((sh2.Kc, sh2.N), dtype=torch.float32, device="cuda"), dx2.t)
    torch.cuda.synchronize()
    assert d4r.d4r_conv_describe(pl2.h)["col2im"] == "gather"
    assert dx.intact() and dx2.intact()
