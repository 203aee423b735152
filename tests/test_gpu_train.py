"""GPU parity of the rest of a training step against the oracle.

Each op of libd4r_conv's training-step entry points (ReLU and its gradient,
max pooling with argmax and its backward, the row bias and its gradient,
softmax and the softmax-cross-entropy gradient with the mean loss, SGD with
clipping, gradient accumulation) runs on seeded float32 inputs and is
compared with the oracle, which computes in float64 from the same float32
values.  Decisions (ReLU masks, max-pool argmax, SGD clipping) depend only
on comparisons of the stored float32 values, which both sides make exactly,
so masks and indices must be identical; sums are compared to a tolerance.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import oracle
import workloads as wl
from gpu_util import host, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-5   # relative Frobenius error of float32 sums against the float64 oracle
EXACT_ELEM = 1e-6  # single-rounding ops: relative error per element


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _f64(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _close_elem(got, ref, rel=EXACT_ELEM):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = rel * np.maximum(np.abs(ref), 1e-30) + 1e-37
    assert np.all(err <= bound), f"max elementwise error {err.max():.3e}"


# ------------------------------------------------------------------ ReLU ----

RELU_SIZES = [1, 3, 4, 1023, 4097, 64 * 6 * 24 * 24, 32 * 96 * 55 * 55 + 3]


@pytest.mark.parametrize("n", RELU_SIZES)
def test_relu_forward_and_gradient_exact(n):
    x = wl.f32_array(("normal", 1.0), (n,), (700, n, 0))
    x[:: 7] = 0.0  # exact zeros: the gradient mask is strict (x > 0)
    dy = wl.f32_array(("normal", 1.0), (n,), (700, n, 1))
    xd, dyd = _dev(x), _dev(dy)
    y = torch.empty_like(xd)
    dx = torch.empty_like(xd)
    d4r.d4r_relu_forward(xd, y, n)
    d4r.d4r_relu_backward(xd, dyd, dx, n)
    torch.cuda.synchronize()
    # one comparison per element: bit-exact
    assert np.array_equal(y.cpu().numpy(), oracle.relu(_f64(x)).astype(np.float32))
    assert np.array_equal(dx.cpu().numpy(), oracle.relu_grad(_f64(x), _f64(dy)).astype(np.float32))


def test_relu_in_place():
    n = 4099
    x = wl.f32_array(("normal", 1.0), (n,), (701, 0))
    dy = wl.f32_array(("normal", 1.0), (n,), (701, 1))
    t = _dev(x)
    d4r.d4r_relu_forward(t, t, n)
    g = _dev(dy)
    d4r.d4r_relu_backward(t, g, g, n)  # mask from the ReLU output: same as from its input
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), oracle.relu(_f64(x)).astype(np.float32))
    assert np.array_equal(g.cpu().numpy(), oracle.relu_grad(_f64(x), _f64(dy)).astype(np.float32))


# ------------------------------------------------------------ max pooling ----

# (batch, channels, H, W, k, stride): LeNet 2x2/2, AlexNet 3x3/2 (overlapping),
# k > stride ragged, stride > k (gaps), k = 1, a window equal to the plane
POOL_CASES = [(64, 6, 24, 24, 2, 2), (64, 16, 8, 8, 2, 2), (8, 96, 55, 55, 3, 2), (3, 5, 13, 11, 3, 1),
              (2, 3, 11, 14, 2, 3), (2, 2, 7, 9, 1, 1), (3, 4, 5, 5, 5, 1), (1, 1, 1, 1, 1, 1),
              (5, 7, 17, 9, 4, 3)]


def _pool_case(case, dist, seed):
    b, c, H, W, k, s = case
    x = wl.f32_array(dist, (b, c, H, W), (702, seed, 0))
    OH, OW = oracle.pool_dims(H, W, k, s)
    dy = wl.f32_array(("normal", 1.0), (b, c, OH, OW), (702, seed, 1))
    return x, dy, OH, OW


def _run_pool(case, x, dy, OH, OW):
    b, c, H, W, k, s = case
    xd, dyd = _dev(x), _dev(dy)
    y = torch.empty((b, c, OH, OW), dtype=torch.float32, device="cuda")
    idx = torch.empty((b, c, OH, OW), dtype=torch.int32, device="cuda")
    dx = torch.full((b, c, H, W), float("nan"), dtype=torch.float32, device="cuda")
    d4r.d4r_maxpool_forward(xd, y, idx, b, c, H, W, k, s)
    d4r.d4r_maxpool_backward(dyd, idx, dx, b, c, H, W, k, s)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), dx.cpu().numpy()


@pytest.mark.parametrize("case", POOL_CASES, ids=[str(c) for c in POOL_CASES])
@pytest.mark.parametrize("dist", [("normal", 1.0), ("small_int", 1)], ids=["normal", "ties"])
def test_maxpool_matches_oracle(case, dist):
    b, c, H, W, k, s = case
    x, dy, OH, OW = _pool_case(case, dist, POOL_CASES.index(case))
    y, idx, dx = _run_pool(case, x, dy, OH, OW)
    ry, ridx = oracle.maxpool_forward(_f64(x), k, s)
    assert np.array_equal(idx, ridx)            # argmax, first maximum on ties
    assert np.array_equal(y, ry.astype(np.float32))
    rdx = oracle.maxpool_backward(_f64(dy), ridx, x.shape, k, s)
    assert np.all(np.isfinite(dx))               # every element written
    assert rel_err(dx, rdx) <= TOL
    if s >= k:  # windows do not overlap: each dx entry is one dy value or 0
        assert np.array_equal(dx, rdx.astype(np.float32))


# ------------------------------------------------------------ row bias -------

BIAS_CASES = [(64, 120), (64, 84), (64, 10), (1, 1), (3, 7), (1000, 65), (4096, 4096), (0, 5), (7, 1)]


@pytest.mark.parametrize("rows,cols", BIAS_CASES)
def test_bias_rows_match_oracle(rows, cols):
    x = wl.f32_array(("normal", 1.0), (rows, cols), (703, rows, cols, 0))
    bias = wl.f32_array(("normal", 0.1), (cols,), (703, rows, cols, 1))
    dy = wl.f32_array(("normal", 1.0), (rows, cols), (703, rows, cols, 2))
    xd = _dev(x)
    y = torch.empty_like(xd)
    db = torch.full((cols,), float("nan"), dtype=torch.float32, device="cuda")
    d4r.d4r_add_bias_rows(xd, _dev(bias), y, rows, cols)
    d4r.d4r_bias_grad_rows(_dev(dy), db, rows, cols)
    # in place on a copy
    t = xd.clone()
    d4r.d4r_add_bias_rows(t, _dev(bias), t, rows, cols)
    torch.cuda.synchronize()
    if rows == 0:  # nothing to add; the gradient is the empty sum
        assert np.array_equal(db.cpu().numpy(), np.zeros(cols, np.float32))
        return
    ref = oracle.add_bias_rows(_f64(x), _f64(bias))
    _close_elem(y.cpu().numpy(), ref)
    assert np.array_equal(t.cpu().numpy(), y.cpu().numpy())
    assert rel_err(host(db), oracle.bias_grad_rows(_f64(dy))) <= TOL


# ------------------------------------------------- softmax cross-entropy -----

# (rows, classes): LeNet 64x10, AlexNet cats/dogs 2, 1000 classes, a single
# class, lane tails (65, 130), more rows than one workgroup has waves
SOFTMAX_CASES = [(64, 10), (64, 2), (32, 1000), (5, 1), (17, 65), (3, 130), (1, 10), (1000, 10), (4096, 37)]


def _logits(rows, classes, seed):
    z = wl.f32_array(("normal", 3.0), (rows, classes), (704, seed, 0))
    lab = wl.labels(rows, classes, (704, seed, 1))
    return z, lab


@pytest.mark.parametrize("rows,classes", SOFTMAX_CASES)
def test_softmax_ce_matches_oracle(rows, classes):
    z, lab = _logits(rows, classes, SOFTMAX_CASES.index((rows, classes)))
    zd, ld = _dev(z), _dev(lab)
    p = torch.empty_like(zd)
    dz = torch.empty_like(zd)
    dz2 = torch.empty_like(zd)
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    d4r.d4r_softmax(zd, p, rows, classes)
    d4r.d4r_softmax_ce_grad(zd, ld, dz, loss, rows, classes)
    d4r.d4r_softmax_ce_grad(zd, ld, dz2, None, rows, classes)  # no loss: one wave per row, many blocks
    torch.cuda.synchronize()
    rp = oracle.softmax(_f64(z))
    assert rel_err(host(p), rp) <= TOL
    _close_elem(host(p).sum(axis=1), np.ones(rows), rel=1e-5)
    rdz = oracle.softmax_ce_grad(_f64(z), lab)
    assert rel_err(host(dz), rdz) <= TOL
    assert np.array_equal(dz.cpu().numpy(), dz2.cpu().numpy())
    rl = oracle.ce_loss(_f64(z), lab)
    assert abs(float(loss.item()) - rl) <= TOL * max(abs(rl), 1e-3)


def test_softmax_ce_loss_is_deterministic():
    z, lab = _logits(4096, 37, 99)
    zd, ld = _dev(z), _dev(lab)
    dz = torch.empty_like(zd)
    losses = []
    for _ in range(3):
        loss = torch.empty((1,), dtype=torch.float32, device="cuda")
        d4r.d4r_softmax_ce_grad(zd, ld, dz, loss, 4096, 37)
        losses.append(loss.cpu().numpy().tobytes())
    assert losses[0] == losses[1] == losses[2]


def test_softmax_ce_bad_label_gives_nan_row():
    z, lab = _logits(8, 10, 7)
    lab[3] = 10   # outside [0, classes)
    lab[5] = -1
    zd, ld = _dev(z), _dev(lab)
    dz = torch.empty_like(zd)
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    d4r.d4r_softmax_ce_grad(zd, ld, dz, loss, 8, 10)
    torch.cuda.synchronize()
    g = dz.cpu().numpy()
    assert np.all(np.isnan(g[3])) and np.all(np.isnan(g[5]))
    good = [0, 1, 2, 4, 6, 7]
    assert rel_err(g[good], oracle.softmax_ce_grad(_f64(z[good]), lab[good])) <= TOL
    assert np.isnan(loss.item())


# -------------------------------------------------- SGD and accumulation -----

SGD_SIZES = [1, 5, 4096, 61706, 1_000_003]


@pytest.mark.parametrize("n", SGD_SIZES)
@pytest.mark.parametrize("clip", [0.5, float("inf"), 0.0])
def test_sgd_matches_oracle(n, clip):
    p = wl.f32_array(("normal", 1.0), (n,), (705, n, 0))
    g = wl.f32_array(("normal", 1.0), (n,), (705, n, 1))
    pd = _dev(p)
    lr = float(np.float32(0.01))  # the value the float32 argument holds
    d4r.d4r_sgd_update(pd, _dev(g), n, lr, clip)
    torch.cuda.synchronize()
    ref = oracle.sgd(_f64(p), _f64(g), lr, clip)
    got = host(pd)
    # p - lr*c(g): the float32 product and difference round twice
    assert np.all(np.abs(got - ref) <= 2 * 2.0 ** -24 * (np.abs(ref) + lr * np.abs(_f64(g))) + 1e-30)
    if clip == 0.0:
        assert np.array_equal(pd.cpu().numpy(), p)


@pytest.mark.parametrize("n", SGD_SIZES)
def test_grad_accum_matches_oracle(n):
    a = wl.f32_array(("normal", 1.0), (n,), (706, n, 0))
    g = wl.f32_array(("normal", 1.0), (n,), (706, n, 1))
    ad = _dev(a)
    d4r.d4r_grad_accum(ad, _dev(g), n)
    torch.cuda.synchronize()
    ref = oracle.grad_accum(_f64(a), _f64(g))
    # one rounding of an exact sum
    assert np.array_equal(ad.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("n", [16, 4096, 1 << 20, (1 << 22) + 48])
def test_stream_reference_kernels(n):
    # the streaming reference kernels: exact copies and fills, tails included
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    d4r.d4r_stream_copy(dst, src, n)
    fill = torch.zeros_like(src)
    d4r.d4r_stream_fill(fill, 0xDEADBEEF, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert bool(torch.all(fill == torch.tensor(0xDEADBEEF, dtype=torch.int64).to(torch.int32).item()))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_mfma_ceiling_closed_form(dt):
    # every operand 1.0: each MFMA adds k (2 for f32, 16 for f16/bf16) to every
    # accumulator element, so each wavefront's sum of its 8 x 16 elements is
    # 128 * k * iters, exactly
    code = {"f32": d4r.D4R_F32, "f16": d4r.D4R_F16, "bf16": d4r.D4R_BF16}[dt]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    per_lane = 1 if dt == "f32" else 8
    src = torch.ones(6 * 64 * per_lane, dtype=tdt, device="cuda")
    blocks, iters = 37, 100
    out = torch.full((blocks * 8,), float("nan"), dtype=torch.float32, device="cuda")
    d4r.d4r_mfma_ceiling(code, src, out, blocks, iters)
    torch.cuda.synchronize()
    k = 2 if dt == "f32" else 16
    assert bool(torch.all(out == 128.0 * k * iters)), out[:8]
