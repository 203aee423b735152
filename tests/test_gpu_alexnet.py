"""A whole AlexNet training step on the GPU against the oracle's step.

The step (gemm_scratch_nn_amd.alexnet.AlexNetStep) issues only library
calls: five convolutions (bias and ReLU in the forward GEMM's epilogue, one
combined backward per layer reusing the saved col), 3x3 / 2 max pooling
with argmax, three linear layers (matmul flags, bias and ReLU in the
epilogue), the softmax-cross-entropy gradient and one SGD launch.  The
oracle (oracle.alexnet_step) composes its float64 routines in the same
order.  Inputs are continuous (U[0,1) images, Kaiming weights), so the GPU's
float32 rounding can only move ReLU and max-pool decisions whose margins are
at rounding level; their effect on the relative Frobenius error of each
gradient stays far below the tolerance used here.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import host, rel_err

pytestmark = pytest.mark.gpu

LR, CLIP = 0.01, 0.002


def _setup(batch, seed):
    from gemm_scratch_nn_amd.alexnet import AlexNetStep
    inp = wl.alexnet_step_inputs(batch, seed)
    net = AlexNetStep(batch)
    net.load({n: torch.from_numpy(inp[n]).cuda() for n, _ in wl.ALEXNET_PARAMS})
    x = torch.from_numpy(inp["x"]).cuda()
    lab = torch.from_numpy(inp["labels"]).cuda()
    return inp, net, x, lab


def test_alexnet_step_matches_oracle():
    inp, net, x, lab = _setup(2, 0)
    r = oracle.alexnet_step(inp, float(np.float32(LR)), CLIP)
    old = net.flat.clone()
    net.forward_backward(x, lab)
    torch.cuda.synchronize()
    acts = {"a1": net.a["conv1"], "p1": net.pool["conv1"][0], "a2": net.a["conv2"], "a3": net.a["conv3"],
            "a5": net.a["conv5"], "p5": net.pool["conv5"][0], "h1": net.h1, "h2": net.h2, "z": net.z,
            "dz": net.dz}
    for k, t in acts.items():
        err = rel_err(host(t), r[k])
        print(f"alexnet {k}: {err:.2e}", flush=True)
        assert err <= 1e-5, k
    assert abs(net.loss.item() - r["loss"]) <= 1e-5 * abs(r["loss"])
    for name, _ in wl.ALEXNET_PARAMS:
        err = rel_err(host(net.g[name]), r["d" + name])
        print(f"alexnet d{name}: {err:.2e}", flush=True)
        assert err <= 1e-5, name
    # the gaps between parameters in the gradient buffer stay zero, and the
    # update leaves them alone
    mask = torch.ones_like(net.flat_grad, dtype=torch.bool)
    for name, shape in wl.ALEXNET_PARAMS:
        o = net.offsets[name]
        mask[o:o + int(np.prod(shape))] = False
    assert not net.flat_grad[mask].any()
    net.update(float(np.float32(LR)), CLIP)
    torch.cuda.synchronize()
    assert torch.equal(net.flat[mask], old[mask])
    for name, _ in wl.ALEXNET_PARAMS:
        assert rel_err(host(net.p[name]), r["new_" + name]) <= 1e-6, name


def test_alexnet_steps_graph_replay_matches_eager():
    _, eager, x, lab = _setup(4, 1)
    _, graphed, _, _ = _setup(4, 1)
    gx, glab = x.clone(), lab.clone()
    graphed.step(gx, glab, LR, CLIP)  # warm up outside capture
    eager.step(x, lab, LR, CLIP)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step(gx, glab, LR, CLIP)
    torch.cuda.synchronize()
    for i in range(3):
        x.copy_(torch.roll(x, shifts=1 + i, dims=3))
        lab.copy_(1 - lab)
        gx.copy_(x)
        glab.copy_(lab)
        torch.cuda.synchronize()
        graph.replay()
        eager.step(x, lab, LR, CLIP)
        torch.cuda.synchronize()
        assert torch.equal(graphed.flat, eager.flat), i
        assert torch.equal(graphed.loss, eager.loss), i
    # training lowers the loss of a repeated batch
    first = eager.loss.item()
    for _ in range(10):
        eager.step(x, lab, LR, CLIP)
    torch.cuda.synchronize()
    assert eager.loss.item() < first
