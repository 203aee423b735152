"""One LeNet-5 training step issued through libd4r_conv's entry points.

The network is the directcompute-nn page's LeNet ("File Structure": 1->6->16
conv, 256->120->84->10 FC) on 1x28x28 images: conv 5x5 (no padding), ReLU,
max pool 2x2 stride 2, twice; flatten to 256; linear 256->120, ReLU,
120->84, ReLU, 84->10; softmax-cross-entropy; SGD with gradient clipping.
The backward follows the page's autograd ("Autograd", "Convolution: The
im2col Approach"): conv gradients by im2col + GEMM (the saved col matrix is
reused for the filter gradient), linear gradients by the matmul flags, the
loss gradient softmax - one_hot.

Each layer's bias and ReLU run in the epilogue of its GEMM (conv forward
with D4R_FWD_RELU, linear layers through d4r_gemm_bias_act), so the
activations are stored once.

Marshalling and sequencing only: every value is computed by a library
kernel.  torch provides the device buffers (allocated once, in the
constructor) and the stream, so a whole step can be captured in a HIP graph
and replayed.  Parameters live in one flat buffer and gradients in another
(each tensor at a 256-byte aligned offset), so the update is one SGD launch
over all parameters; the gaps between tensors hold zeros in the gradient
buffer and are left unchanged by the update.
"""
from __future__ import annotations

from typing import Dict

import torch

from . import (ConvPlan, D4R_F32, d4r_bias_grad_rows, d4r_gemm, d4r_gemm_bias_act,
               d4r_gemm_workspace_size, d4r_maxpool_backward, d4r_maxpool_forward,
               d4r_relu_backward, d4r_sgd_update, d4r_softmax_ce_grad)

PARAMS = (("conv1_w", (6, 1, 5, 5)), ("conv1_b", (6,)),
          ("conv2_w", (16, 6, 5, 5)), ("conv2_b", (16,)),
          ("fc1_w", (120, 256)), ("fc1_b", (120,)),
          ("fc2_w", (84, 120)), ("fc2_b", (84,)),
          ("fc3_w", (10, 84)), ("fc3_b", (10,)))

_ALIGN = 64  # floats: 256 bytes


def _numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n


class LeNetStep:
    """Buffers and the call sequence of one LeNet-5 training step (float32)."""

    def __init__(self, batch: int, device="cuda"):
        if batch < 1:
            raise ValueError("batch must be >= 1")
        self.batch = B = batch
        dev = torch.device(device)
        f32 = dict(dtype=torch.float32, device=dev)
        # flat parameter and gradient buffers
        self.offsets: Dict[str, int] = {}
        off = 0
        for name, shape in PARAMS:
            self.offsets[name] = off
            off += (_numel(shape) + _ALIGN - 1) // _ALIGN * _ALIGN
        self.n_flat = off
        self.flat = torch.zeros(off, **f32)
        self.flat_grad = torch.zeros(off, **f32)
        self.p = {n: self.flat[self.offsets[n]:self.offsets[n] + _numel(s)].view(s) for n, s in PARAMS}
        self.g = {n: self.flat_grad[self.offsets[n]:self.offsets[n] + _numel(s)].view(s) for n, s in PARAMS}
        # convolutions (each keeps its own workspace; the forward's col matrix
        # stays there for the filter gradient)
        self.c1 = ConvPlan(B, 1, 28, 28, 5, 5, 1, 0, 6, D4R_F32, device=dev)
        self.c2 = ConvPlan(B, 6, 12, 12, 5, 5, 1, 0, 16, D4R_F32, device=dev)
        # activations (a1, a2 hold the ReLU outputs in place of the conv outputs)
        self.a1 = torch.empty((B, 6, 24, 24), **f32)
        self.p1 = torch.empty((B, 6, 12, 12), **f32)
        self.idx1 = torch.empty((B, 6, 12, 12), dtype=torch.int32, device=dev)
        self.a2 = torch.empty((B, 16, 8, 8), **f32)
        self.p2 = torch.empty((B, 16, 4, 4), **f32)
        self.idx2 = torch.empty((B, 16, 4, 4), dtype=torch.int32, device=dev)
        self.h1 = torch.empty((B, 120), **f32)
        self.h2 = torch.empty((B, 84), **f32)
        self.z = torch.empty((B, 10), **f32)
        self.loss = torch.empty((1,), **f32)
        # gradients of activations
        self.dz = torch.empty((B, 10), **f32)
        self.dh2 = torch.empty((B, 84), **f32)
        self.dh1 = torch.empty((B, 120), **f32)
        self.dflat = torch.empty((B, 256), **f32)
        self.da2 = torch.empty((B, 16, 8, 8), **f32)
        self.dp1 = torch.empty((B, 6, 12, 12), **f32)
        self.da1 = torch.empty((B, 6, 24, 24), **f32)
        # one split-K workspace for every linear-layer GEMM
        self._gemms = [(B, 256, 120, 2), (B, 120, 84, 2), (B, 84, 10, 2),
                       (10, B, 84, 1), (B, 10, 84, 0), (84, B, 120, 1), (B, 84, 120, 0),
                       (120, B, 256, 1), (B, 120, 256, 0)]
        wsb = max(d4r_gemm_workspace_size(M, K, N, fl, D4R_F32) for M, K, N, fl in self._gemms)
        self.gws_bytes = wsb
        self.gws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def load(self, params: Dict[str, torch.Tensor]) -> None:
        """Copy parameter values (tensors of the PARAMS shapes) into the flat buffer."""
        for name, shape in PARAMS:
            t = params[name]
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
            self.p[name].copy_(t)

    def _gemm(self, M, K, N, flags, A, Bm, C):
        d4r_gemm(M, K, N, flags, D4R_F32, A, Bm, C, self.gws, self.gws_bytes)

    def _linear(self, M, K, N, x, w, b, relu, out):
        # out = x * w^T + b (then ReLU): matmul flags 2 with the fused epilogue
        d4r_gemm_bias_act(M, K, N, 2, D4R_F32, x, w, b, relu, out, self.gws, self.gws_bytes)

    def forward_backward(self, x: torch.Tensor, labels: torch.Tensor) -> None:
        """Loss, every gradient (into flat_grad) for one batch; no update."""
        B, p, g = self.batch, self.p, self.g
        if tuple(x.shape) != (B, 1, 28, 28) or x.dtype != torch.float32:
            raise ValueError("x must be float32 of shape (batch, 1, 28, 28)")
        if tuple(labels.shape) != (B,) or labels.dtype != torch.int32:
            raise ValueError("labels must be int32 of shape (batch,)")
        # forward (the conv forwards keep col in their workspaces)
        self.c1.forward_relu(x, p["conv1_w"], p["conv1_b"], y=self.a1)
        d4r_maxpool_forward(self.a1, self.p1, self.idx1, B, 6, 24, 24, 2, 2)
        self.c2.forward_relu(self.p1, p["conv2_w"], p["conv2_b"], y=self.a2)
        d4r_maxpool_forward(self.a2, self.p2, self.idx2, B, 16, 8, 8, 2, 2)
        self._linear(B, 256, 120, self.p2, p["fc1_w"], p["fc1_b"], 1, self.h1)
        self._linear(B, 120, 84, self.h1, p["fc2_w"], p["fc2_b"], 1, self.h2)
        self._linear(B, 84, 10, self.h2, p["fc3_w"], p["fc3_b"], 0, self.z)
        # loss gradient
        d4r_softmax_ce_grad(self.z, labels, self.dz, self.loss, B, 10)
        # fc3, fc2, fc1 (ReLU masks from the stored ReLU outputs)
        self._gemm(10, B, 84, 1, self.dz, self.h2, g["fc3_w"])
        d4r_bias_grad_rows(self.dz, g["fc3_b"], B, 10)
        self._gemm(B, 10, 84, 0, self.dz, p["fc3_w"], self.dh2)
        d4r_relu_backward(self.h2, self.dh2, self.dh2, self.dh2.numel())
        self._gemm(84, B, 120, 1, self.dh2, self.h1, g["fc2_w"])
        d4r_bias_grad_rows(self.dh2, g["fc2_b"], B, 84)
        self._gemm(B, 84, 120, 0, self.dh2, p["fc2_w"], self.dh1)
        d4r_relu_backward(self.h1, self.dh1, self.dh1, self.dh1.numel())
        self._gemm(120, B, 256, 1, self.dh1, self.p2, g["fc1_w"])
        d4r_bias_grad_rows(self.dh1, g["fc1_b"], B, 120)
        self._gemm(B, 120, 256, 0, self.dh1, p["fc1_w"], self.dflat)
        # pool2, conv2 (data gradient first: it leaves the saved col matrix intact)
        d4r_maxpool_backward(self.dflat, self.idx2, self.da2, B, 16, 8, 8, 2, 2)
        d4r_relu_backward(self.a2, self.da2, self.da2, self.da2.numel())
        self.c2.backward_data(p["conv2_w"], self.da2, dx=self.dp1)
        self.c2.backward_filter(None, self.da2, reuse_col=True, dw=g["conv2_w"], db=g["conv2_b"])
        # pool1, conv1 (no data gradient for the input image)
        d4r_maxpool_backward(self.dp1, self.idx1, self.da1, B, 6, 24, 24, 2, 2)
        d4r_relu_backward(self.a1, self.da1, self.da1, self.da1.numel())
        self.c1.backward_filter(None, self.da1, reuse_col=True, dw=g["conv1_w"], db=g["conv1_b"])

    def update(self, lr: float, clip: float) -> None:
        """param -= lr * clamp(grad, -clip, clip) over every parameter (one launch)."""
        d4r_sgd_update(self.flat, self.flat_grad, self.n_flat, lr, clip)

    def step(self, x: torch.Tensor, labels: torch.Tensor, lr: float, clip: float) -> None:
        self.forward_backward(x, labels)
        self.update(lr, clip)
