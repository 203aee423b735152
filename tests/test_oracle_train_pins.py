"""Pins of the oracle's training-step routines (CPU only).

The directcompute-nn page lists these operations in its "HLSL Shader
Reference" ("Activation / Loss Shaders", "Pooling Shaders", "Utility
Shaders").  Each routine is checked against something other than itself:
torch float64 operators and autograd, closed forms, adjoint identities and
finite differences; tie handling of the max-pool argmax against a
hand-worked fixture.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _t(a):
    return torch.tensor(np.asarray(a), dtype=torch.float64)


# ---------------------------------------------------------------- ReLU
def test_relu_values_and_gradient_at_zero(orc):
    x = np.array([-2.0, -0.0, 0.0, 1e-300, 3.5])
    assert np.array_equal(orc.relu(x), [0.0, 0.0, 0.0, 1e-300, 3.5])
    dy = np.array([1.0, 2.0, 3.0, 4.0, 5.0])
    # reading: gradient only where x > 0 strictly
    assert np.array_equal(orc.relu_grad(x, dy), [0.0, 0.0, 0.0, 4.0, 5.0])


def test_relu_matches_torch_autograd(orc):
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 4, 5, 6))
    g = rng.normal(size=x.shape)
    xt = _t(x).requires_grad_()
    y = F.relu(xt)
    y.backward(_t(g))
    assert np.array_equal(orc.relu(x), y.detach().numpy())
    assert np.array_equal(orc.relu_grad(x, g), xt.grad.numpy())


# ---------------------------------------------------------------- max pooling
@pytest.mark.parametrize("shape,k,s", [((2, 3, 8, 8), 2, 2), ((2, 3, 9, 7), 2, 2), ((1, 4, 13, 13), 3, 2),
                                       ((2, 2, 11, 10), 3, 3), ((1, 1, 5, 5), 5, 1), ((2, 2, 6, 9), 1, 2)])
def test_maxpool_matches_torch(orc, shape, k, s):
    rng = np.random.default_rng(sum(shape) + k + s)
    x = rng.permutation(np.prod(shape)).reshape(shape).astype(np.float64)  # distinct values
    g = rng.normal(size=(shape[0], shape[1]) + orc.pool_dims(shape[2], shape[3], k, s))
    xt = _t(x).requires_grad_()
    yt, it = F.max_pool2d(xt, k, s, return_indices=True)
    yt.backward(_t(g))
    y, idx = orc.maxpool_forward(x, k, s)
    assert np.array_equal(y, yt.detach().numpy())
    assert np.array_equal(idx, it.numpy())
    assert np.array_equal(orc.maxpool_backward(g, idx, shape, k, s), xt.grad.numpy())


def test_maxpool_backward_is_the_selection_adjoint(orc):
    # y = S x for the saved selection S, so <y, g> = <x, S^T g> exactly on
    # small integers, overlapping windows included
    rng = np.random.default_rng(5)
    x = rng.integers(-50, 50, size=(2, 3, 13, 13)).astype(np.float64)
    y, idx = orc.maxpool_forward(x, 3, 2)
    g = rng.integers(-9, 9, size=y.shape).astype(np.float64)
    dx = orc.maxpool_backward(g, idx, x.shape, 3, 2)
    assert float(np.vdot(y, g)) == float(np.vdot(x, dx))
    # every saved index points at the value it reports
    planes = x.reshape(6, -1)
    assert np.array_equal(np.take_along_axis(planes, idx.reshape(6, -1), 1).reshape(y.shape), y)


def test_maxpool_ties_take_the_first_maximum(orc):
    x = np.full((1, 2, 4, 6), 7.0)
    y, idx = orc.maxpool_forward(x, 2, 2)
    H, W = 4, 6
    want = np.array([[h * W + w for w in range(0, W, 2)] for h in range(0, H, 2)])
    assert np.array_equal(idx[0, 0], want) and np.array_equal(idx[0, 1], want)
    assert np.all(y == 7.0)


def test_maxpool_golden_fixture(orc):
    with open(os.path.join(GOLDEN, "maxpool_handworked_ties.json")) as f:
        fx = json.load(f)
    x = np.array(fx["x"], dtype=np.float64)
    y, idx = orc.maxpool_forward(x, fx["k"], fx["s"])
    assert np.array_equal(y, np.array(fx["y"])) and np.array_equal(idx, np.array(fx["idx"]))
    dx = orc.maxpool_backward(np.array(fx["dy"], dtype=np.float64), idx, x.shape, fx["k"], fx["s"])
    assert np.array_equal(dx, np.array(fx["dx"]))


def test_maxpool_rejects_windows_larger_than_the_plane(orc):
    with pytest.raises(ValueError):
        orc.maxpool_forward(np.zeros((1, 1, 3, 3)), 4, 1)


# ---------------------------------------------------------------- bias rows
def test_bias_rows_closed_forms_and_adjoint(orc):
    rng = np.random.default_rng(7)
    b = rng.normal(size=5)
    assert np.array_equal(orc.add_bias_rows(np.zeros((3, 5)), b), np.tile(b, (3, 1)))
    assert np.array_equal(orc.bias_grad_rows(np.ones((4, 3))), [4.0, 4.0, 4.0])
    g = rng.integers(-9, 9, size=(6, 5)).astype(np.float64)
    bi = rng.integers(-9, 9, size=5).astype(np.float64)
    # <add_bias(0, b), g> = <b, bias_grad(g)>
    assert float(np.vdot(orc.add_bias_rows(np.zeros((6, 5)), bi), g)) == \
        float(np.vdot(bi, orc.bias_grad_rows(g)))
    x = rng.normal(size=(6, 5))
    xt = _t(x).requires_grad_()
    bt = _t(b).requires_grad_()
    (xt + bt).backward(_t(g))
    assert np.allclose(orc.add_bias_rows(x, b), (xt + bt).detach().numpy(), rtol=0, atol=0)
    assert np.allclose(orc.bias_grad_rows(g), bt.grad.numpy(), rtol=1e-15, atol=0)


# ---------------------------------------------------------------- softmax / CE
def test_softmax_closed_forms(orc):
    p = orc.softmax(np.zeros((3, 10)))
    assert np.allclose(p, 0.1, rtol=1e-15)
    rng = np.random.default_rng(9)
    z = rng.normal(size=(5, 7)) * 30
    p = orc.softmax(z)
    assert np.allclose(p.sum(1), 1.0, rtol=1e-14)
    assert np.allclose(orc.softmax(z + 123.0), p, rtol=1e-12)   # shift invariance
    assert np.allclose(p, torch.softmax(_t(z), 1).numpy(), rtol=1e-13, atol=1e-300)


def test_ce_loss_closed_form_and_torch(orc):
    assert abs(orc.ce_loss(np.zeros((4, 10)), [0, 3, 9, 5]) - np.log(10)) < 1e-15
    rng = np.random.default_rng(11)
    z = rng.normal(size=(8, 10)) * 3
    lab = rng.integers(0, 10, size=8)
    ref = F.cross_entropy(_t(z), torch.tensor(lab), reduction="mean").item()
    assert abs(orc.ce_loss(z, lab) - ref) < 1e-13


def test_softmax_ce_grad_is_the_loss_derivative(orc):
    rng = np.random.default_rng(13)
    z = rng.normal(size=(4, 10))
    lab = rng.integers(0, 10, size=4)
    d = orc.softmax_ce_grad(z, lab)
    assert np.allclose(d.sum(1), 0.0, atol=1e-15)
    zt = _t(z).requires_grad_()
    F.cross_entropy(zt, torch.tensor(lab), reduction="sum").backward()
    assert np.allclose(d, zt.grad.numpy(), rtol=1e-13, atol=1e-15)
    # central differences of rows * mean loss
    eps = 1e-6
    fd = np.empty_like(z)
    for i in range(z.shape[0]):
        for j in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += eps
            zm[i, j] -= eps
            fd[i, j] = (orc.ce_loss(zp, lab) - orc.ce_loss(zm, lab)) * z.shape[0] / (2 * eps)
    assert np.allclose(d, fd, rtol=0, atol=1e-8)


def test_ce_rejects_out_of_range_labels(orc):
    with pytest.raises(ValueError):
        orc.softmax_ce_grad(np.zeros((2, 3)), [0, 3])


# ---------------------------------------------------------------- SGD / accumulation
def test_sgd_clips_both_sides(orc):
    p = np.array([1.0, 1.0, 1.0, 1.0, 1.0])
    g = np.array([-10.0, -0.5, 0.0, 0.25, 8.0])
    assert np.array_equal(orc.sgd(p, g, lr=0.5, clip=1.0), [1.5, 1.25, 1.0, 0.875, 0.5])
    assert np.array_equal(orc.sgd(p, g, lr=0.5, clip=np.inf), [6.0, 1.25, 1.0, 0.875, -3.0])


def test_grad_accum_adds(orc):
    assert np.array_equal(orc.grad_accum([1.0, -2.0, 0.5], [0.25, 2.0, -0.5]), [1.25, 0.0, 0.0])


# ---------------------------------------------------- a whole LeNet-5 step
def _lenet_torch_f64(inp, lr, clip):
    """The same network in torch float64 autograd (independent operators)."""
    p = {k: _t(v).requires_grad_() for k, v in inp.items() if k not in ("x", "labels")}
    x = _t(inp["x"])
    a = F.max_pool2d(F.relu(F.conv2d(x, p["conv1_w"], p["conv1_b"])), 2, 2)
    a = F.max_pool2d(F.relu(F.conv2d(a, p["conv2_w"], p["conv2_b"])), 2, 2)
    h = a.reshape(a.shape[0], -1)
    h = F.relu(F.linear(h, p["fc1_w"], p["fc1_b"]))
    h = F.relu(F.linear(h, p["fc2_w"], p["fc2_b"]))
    z = F.linear(h, p["fc3_w"], p["fc3_b"])
    lab = torch.tensor(inp["labels"], dtype=torch.long)
    # the page's loss gradient is softmax - one_hot per row: the gradient of
    # the summed (not averaged) cross-entropy
    F.cross_entropy(z, lab, reduction="sum").backward()
    loss = F.cross_entropy(z, lab).item()
    new = {k: (v - lr * torch.clamp(v.grad, -clip, clip)).detach().numpy() for k, v in p.items()}
    return loss, {k: v.grad.numpy() for k, v in p.items()}, new


@pytest.mark.parametrize("batch,seed", [(8, 0), (3, 1)])
def test_lenet_step_matches_torch_autograd(orc, batch, seed):
    import workloads as wl
    rng = np.random.default_rng((880, seed))
    inp = {"x": rng.uniform(0.0, 1.0, size=(batch, 1, 28, 28)),
           "labels": rng.integers(0, 10, size=batch).astype(np.int32)}
    for name, shape in wl.LENET_PARAMS:  # continuous values: no max-pool ties
        inp[name] = rng.normal(0.0, 0.3, size=shape)
    lr, clip = 0.05, 0.02
    r = orc.lenet_step(inp, lr, clip)
    loss, grads, new = _lenet_torch_f64(inp, lr, clip)
    assert abs(r["loss"] - loss) <= 1e-12 * max(1.0, abs(loss))
    for name, g in grads.items():
        assert np.allclose(r["d" + name], g, rtol=1e-10, atol=1e-12), name
        assert np.allclose(r["new_" + name], new[name], rtol=1e-12, atol=1e-14), name
    # the clip acted on some gradients and not on others
    d = np.concatenate([np.abs(g).ravel() for g in grads.values()])
    assert (d > clip).any() and (d < clip).any()


# ---------------------------------------------------- a whole AlexNet step
def _alexnet_torch_f64(inp, lr, clip):
    """The same network in torch float64 autograd (independent operators)."""
    p = {k: _t(v).requires_grad_() for k, v in inp.items() if k not in ("x", "labels")}
    a = _t(inp["x"])
    for name, s, pad, pool in (("conv1", 4, 2, True), ("conv2", 1, 2, True), ("conv3", 1, 1, False),
                               ("conv4", 1, 1, False), ("conv5", 1, 1, True)):
        a = F.relu(F.conv2d(a, p[name + "_w"], p[name + "_b"], stride=s, padding=pad))
        if pool:
            a = F.max_pool2d(a, 3, 2)
    h = a.reshape(a.shape[0], -1)
    h = F.relu(F.linear(h, p["fc1_w"], p["fc1_b"]))
    h = F.relu(F.linear(h, p["fc2_w"], p["fc2_b"]))
    z = F.linear(h, p["fc3_w"], p["fc3_b"])
    lab = torch.tensor(inp["labels"], dtype=torch.long)
    F.cross_entropy(z, lab, reduction="sum").backward()
    loss = F.cross_entropy(z, lab).item()
    new = {k: (v - lr * torch.clamp(v.grad, -clip, clip)).detach().numpy() for k, v in p.items()}
    return loss, {k: v.grad.numpy() for k, v in p.items()}, new


def test_alexnet_step_matches_torch_autograd(orc):
    # the oracle's AlexNet composition (layer order, strides, paddings,
    # pools, flatten, linear flags) on a smaller input and hidden width, so
    # its float64 loops stay fast: 3x99x99 -> conv1 24x24 -> pool 11 ->
    # conv2 11 -> pool 5 -> conv3-5 5 -> pool 2 -> flatten 1024 -> 256 -> 256
    # -> 2; the same code runs at 224x224 in the GPU parity test.
    # Continuous inputs: no ReLU zeros or max-pool ties.
    import workloads as wl
    rng = np.random.default_rng((881, 0))
    inp = {"x": rng.uniform(0.0, 1.0, size=(2, 3, 99, 99)),
           "labels": np.array([1, 0], dtype=np.int32)}
    shapes = dict(wl.ALEXNET_PARAMS)
    shapes.update({"fc1_w": (256, 1024), "fc1_b": (256,), "fc2_w": (256, 256), "fc2_b": (256,),
                   "fc3_w": (2, 256)})
    for name, shape in shapes.items():
        fan_in = int(np.prod(shape[1:]))
        inp[name] = rng.normal(0.0, np.sqrt(2.0 / fan_in) if name.endswith("_w") else 0.05, size=shape)
    lr, clip = 0.05, 0.002
    r = orc.alexnet_step(inp, lr, clip)
    loss, grads, new = _alexnet_torch_f64(inp, lr, clip)
    assert abs(r["loss"] - loss) <= 1e-10 * max(1.0, abs(loss))
    for name, g in grads.items():
        scale = np.max(np.abs(g))
        assert np.allclose(r["d" + name], g, rtol=1e-8, atol=1e-10 * scale), name
        assert np.allclose(r["new_" + name], new[name], rtol=1e-10, atol=1e-14), name
    d = np.concatenate([np.abs(g).ravel() for g in grads.values()])
    assert (d > clip).any() and (d < clip).any()
