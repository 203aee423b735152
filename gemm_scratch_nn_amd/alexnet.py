"""One AlexNet training step issued through libd4r_conv's entry points.

The network is the one the directcompute-nn page trains on two-class
PetImages ("File Structure": 5 conv layers, 3 FC layers), with the layer
sizes of the AlexNet conv1 and conv3-5 configs: conv1 3->96 11x11 stride 4
pad 2 (224 -> 55), ReLU, max pool 3x3 stride 2; conv2 96->256 5x5 pad 2,
ReLU, pool; conv3 256->384, conv4 384->384, conv5 384->256 (3x3 pad 1) with
ReLU after each and a pool after conv5; flatten to 9216; linear
9216->4096, ReLU, 4096->4096, ReLU, 4096->2; softmax-cross-entropy; SGD
with gradient clipping.

Every conv forward stores relu(conv + bias) from its GEMM epilogue and keeps
its col matrix in the layer's workspace; every conv backward is one
d4r_conv_backward call (data, filter and bias gradients, the saved col
reused), conv1's without the data gradient.  The linear layers use the
matmul flags with bias and ReLU in the epilogue.  Marshalling and
sequencing only: torch provides the buffers (allocated once) and the
stream, so a step can be captured in a HIP graph.  Parameters live in one
flat buffer and gradients in another (256-byte aligned offsets), so the
update is one SGD launch.
"""
from __future__ import annotations

from typing import Dict

import torch

from . import (ConvPlan, D4R_F32, d4r_bias_grad_rows, d4r_gemm, d4r_gemm_bias_act,
               d4r_gemm_workspace_size, d4r_maxpool_backward, d4r_maxpool_forward,
               d4r_relu_backward, d4r_sgd_update, d4r_softmax_ce_grad)

CLASSES = 2
PARAMS = (("conv1_w", (96, 3, 11, 11)), ("conv1_b", (96,)),
          ("conv2_w", (256, 96, 5, 5)), ("conv2_b", (256,)),
          ("conv3_w", (384, 256, 3, 3)), ("conv3_b", (384,)),
          ("conv4_w", (384, 384, 3, 3)), ("conv4_b", (384,)),
          ("conv5_w", (256, 384, 3, 3)), ("conv5_b", (256,)),
          ("fc1_w", (4096, 9216)), ("fc1_b", (4096,)),
          ("fc2_w", (4096, 4096)), ("fc2_b", (4096,)),
          ("fc3_w", (CLASSES, 4096)), ("fc3_b", (CLASSES,)))

# (name, in channels, in size, out channels, kernel, stride, padding, pool after)
CONVS = (("conv1", 3, 224, 96, 11, 4, 2, True),
         ("conv2", 96, 27, 256, 5, 1, 2, True),
         ("conv3", 256, 13, 384, 3, 1, 1, False),
         ("conv4", 384, 13, 384, 3, 1, 1, False),
         ("conv5", 384, 13, 256, 3, 1, 1, True))

_ALIGN = 64  # floats: 256 bytes


def _numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n


class AlexNetStep:
    """Buffers and the call sequence of one AlexNet training step (float32)."""

    def __init__(self, batch: int, device="cuda"):
        if batch < 1:
            raise ValueError("batch must be >= 1")
        self.batch = B = batch
        dev = torch.device(device)
        f32 = dict(dtype=torch.float32, device=dev)
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
        # per conv layer: its plan (own workspace: the forward's col stays
        # there for the filter gradient), ReLU output a, its gradient da,
        # and, after pooled layers, the pooled output, argmax and gradient
        self.plans, self.a, self.da, self.pool = {}, {}, {}, {}
        for name, cin, size, cout, k, s, p, pool in CONVS:
            pl = ConvPlan(B, cin, size, size, k, k, s, p, cout, D4R_F32, device=dev)
            self.plans[name] = pl
            self.a[name] = torch.empty(pl.y_shape, **f32)
            self.da[name] = torch.empty(pl.y_shape, **f32)
            if pool:
                oh = (pl.outH - 3) // 2 + 1
                self.pool[name] = (torch.empty((B, cout, oh, oh), **f32),
                                   torch.empty((B, cout, oh, oh), dtype=torch.int32, device=dev),
                                   torch.empty((B, cout, oh, oh), **f32))
        # the gradient w.r.t. conv1's pooled output is conv2's data gradient
        # (in pool["conv1"][2]); conv1 needs no data gradient
        self.h1 = torch.empty((B, 4096), **f32)
        self.h2 = torch.empty((B, 4096), **f32)
        self.z = torch.empty((B, CLASSES), **f32)
        self.loss = torch.empty((1,), **f32)
        self.dz = torch.empty((B, CLASSES), **f32)
        self.dh2 = torch.empty((B, 4096), **f32)
        self.dh1 = torch.empty((B, 4096), **f32)
        self.dflat = torch.empty((B, 9216), **f32)
        self._gemms = [(B, 9216, 4096, 2), (B, 4096, 4096, 2), (B, 4096, CLASSES, 2),
                       (CLASSES, B, 4096, 1), (B, CLASSES, 4096, 0), (4096, B, 4096, 1), (B, 4096, 4096, 0),
                       (4096, B, 9216, 1), (B, 4096, 9216, 0)]
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
        if tuple(x.shape) != (B, 3, 224, 224) or x.dtype != torch.float32:
            raise ValueError("x must be float32 of shape (batch, 3, 224, 224)")
        if tuple(labels.shape) != (B,) or labels.dtype != torch.int32:
            raise ValueError("labels must be int32 of shape (batch,)")
        # forward
        src = x
        for name, cin, size, cout, k, s, pad, pool in CONVS:
            pl = self.plans[name]
            pl.forward_relu(src, p[name + "_w"], p[name + "_b"], y=self.a[name])
            src = self.a[name]
            if pool:
                y, idx, _ = self.pool[name]
                d4r_maxpool_forward(src, y, idx, B, cout, pl.outH, pl.outW, 3, 2)
                src = y
        self._linear(B, 9216, 4096, src, p["fc1_w"], p["fc1_b"], 1, self.h1)
        self._linear(B, 4096, 4096, self.h1, p["fc2_w"], p["fc2_b"], 1, self.h2)
        self._linear(B, 4096, CLASSES, self.h2, p["fc3_w"], p["fc3_b"], 0, self.z)
        d4r_softmax_ce_grad(self.z, labels, self.dz, self.loss, B, CLASSES)
        # linear layers (ReLU masks from the stored ReLU outputs)
        self._gemm(CLASSES, B, 4096, 1, self.dz, self.h2, g["fc3_w"])
        d4r_bias_grad_rows(self.dz, g["fc3_b"], B, CLASSES)
        self._gemm(B, CLASSES, 4096, 0, self.dz, p["fc3_w"], self.dh2)
        d4r_relu_backward(self.h2, self.dh2, self.dh2, self.dh2.numel())
        self._gemm(4096, B, 4096, 1, self.dh2, self.h1, g["fc2_w"])
        d4r_bias_grad_rows(self.dh2, g["fc2_b"], B, 4096)
        self._gemm(B, 4096, 4096, 0, self.dh2, p["fc2_w"], self.dh1)
        d4r_relu_backward(self.h1, self.dh1, self.dh1, self.dh1.numel())
        self._gemm(4096, B, 9216, 1, self.dh1, self.pool["conv5"][0], g["fc1_w"])
        d4r_bias_grad_rows(self.dh1, g["fc1_b"], B, 4096)
        self._gemm(B, 4096, 9216, 0, self.dh1, p["fc1_w"], self.dflat)
        # conv layers, top down: the gradient reaching each ReLU output, its
        # mask, then one combined backward (the saved col reused)
        d_top = self.dflat
        for i in range(len(CONVS) - 1, -1, -1):
            name, cin, size, cout, k, s, pad, pool = CONVS[i]
            pl = self.plans[name]
            if pool:
                # d_top is the gradient w.r.t. the pooled output
                _, idx, _ = self.pool[name]
                d4r_maxpool_backward(d_top, idx, self.da[name], B, cout, pl.outH, pl.outW, 3, 2)
            # (unpooled: the layer above wrote its data gradient into da[name])
            d4r_relu_backward(self.a[name], self.da[name], self.da[name], self.da[name].numel())
            if i == 0:
                pl.backward_filter(None, self.da[name], reuse_col=True, dw=g[name + "_w"], db=g[name + "_b"])
                break
            prev = CONVS[i - 1]
            # the data gradient lands where the layer below reads it: that
            # layer's pooled-gradient buffer, or its ReLU-gradient buffer
            dx = self.pool[prev[0]][2] if prev[7] else self.da[prev[0]]
            pl.backward(None, p[name + "_w"], self.da[name], reuse_col=True, dx=dx, dw=g[name + "_w"],
                        db=g[name + "_b"])
            d_top = dx

    def update(self, lr: float, clip: float) -> None:
        """param -= lr * clamp(grad, -clip, clip) over every parameter (one launch)."""
        d4r_sgd_update(self.flat, self.flat_grad, self.n_flat, lr, clip)

    def step(self, x: torch.Tensor, labels: torch.Tensor, lr: float, clip: float) -> None:
        self.forward_backward(x, labels)
        self.update(lr, clip)
