"""Seeded synthetic inputs for the five convolution workloads.

This module is shared by the tests, the bench and the smoke check.  It holds
shapes, value distributions and a seeded random generator, and nothing of the
convolution arithmetic itself: no im2col, no GEMM, no reduction.

Workload shapes come from the pages:

* LeNet conv1/conv2 and the 256->120->84 fully connected layers: the
  directcompute-nn page, "File Structure" (train_lenet.py: 1->6->16 conv,
  256->120->84->10 FC).
* AlexNet conv1 and conv3-5: the same page, "Running" / "File Structure"
  (train_alexnet.py, 224x224 inputs, 5 conv layers).  The page prints no
  filter sizes; the classic AlexNet sizes are used (11x11 s4 p2 -> 55x55;
  3x3 p1 at 13x13 with 256/384/384/256 channels).
* The 256x46x80 feature map, its 1x1 256->128 conv and the stride-2 conv to
  the 23x40 latent plane: the mlvc.cpp design page, "ONNX IO" and "Key
  dimensions for 640x368".

Random draws: ``numpy.random.default_rng((cfg, layer, tensor))`` with tensor
ids x=0, W=1, b=2, g=3, A=4, B=5.  Values are drawn in float64, cast to
float32, then rounded to nearest-even to float16 (numpy's cast) or bfloat16
(rounding of the float32 bit pattern).  "N(0, s)" takes s as the standard
deviation; Kaiming-normal is N(0, sqrt(2/fan_in)).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")

TID_X, TID_W, TID_B, TID_G, TID_A, TID_BM = 0, 1, 2, 3, 4, 5


def out_dim(n: int, k: int, s: int, p: int) -> int:
    """Output extent with floor rounding; 0 when the kernel does not fit."""
    span = n + 2 * p - k
    if span < 0:
        return 0
    return span // s + 1


@dataclass(frozen=True)
class ConvShape:
    batch: int
    inC: int
    inH: int
    inW: int
    kH: int
    kW: int
    stride: int
    padding: int
    outC: int

    @property
    def outH(self) -> int:
        return out_dim(self.inH, self.kH, self.stride, self.padding)

    @property
    def outW(self) -> int:
        return out_dim(self.inW, self.kW, self.stride, self.padding)

    @property
    def P(self) -> int:
        return self.outH * self.outW

    @property
    def Kc(self) -> int:
        return self.inC * self.kH * self.kW

    @property
    def N(self) -> int:
        return self.batch * self.P

    def gemm_flops(self) -> int:
        """Flops of one of the three GEMMs (2*O*Kc*N)."""
        return 2 * self.outC * self.Kc * self.N

    def x_shape(self):
        return (self.batch, self.inC, self.inH, self.inW)

    def w_shape(self):
        return (self.outC, self.inC, self.kH, self.kW)

    def y_shape(self):
        return (self.batch, self.outC, self.outH, self.outW)

    def with_batch(self, b: int) -> "ConvShape":
        return ConvShape(b, self.inC, self.inH, self.inW, self.kH, self.kW,
                         self.stride, self.padding, self.outC)


# Distribution specs: ("uniform", lo, hi), ("normal", std), ("relu_normal",)
@dataclass(frozen=True)
class ConvLayer:
    name: str
    shape: ConvShape
    x_dist: tuple
    w_dist: tuple
    b_dist: tuple = ("normal", 0.01)
    g_dist: tuple = ("normal", 1.0)


@dataclass(frozen=True)
class GemmCase:
    name: str
    M: int
    K: int
    N: int
    flags: int
    a_dist: tuple
    b_dist: tuple


@dataclass(frozen=True)
class Workload:
    key: str
    cfg_id: int
    title: str
    dtypes: Tuple[str, ...]
    layers: Tuple[ConvLayer, ...]
    gemms: Tuple[GemmCase, ...] = field(default_factory=tuple)


def _kaiming(fan_in: int) -> tuple:
    return ("normal", float(np.sqrt(2.0 / fan_in)))


def _fc_cases() -> Tuple[GemmCase, ...]:
    cases: List[GemmCase] = []
    # Logical products X[64 x in] * W[in x out]; the flag only changes how an
    # operand is stored (transposed storage for NT / TN).
    for (m, k, n, tag) in ((64, 256, 120, "fc1"), (64, 120, 84, "fc2")):
        for flags, fl in ((0, "nn"), (2, "nt"), (1, "tn")):
            cases.append(GemmCase(f"{tag}_{fl}", m, k, n, flags,
                                  ("normal", 1.0), _kaiming(k)))
    # Linear-layer backward shapes: dX = g * W^T (NT) and dW = X^T * g (TN).
    cases.append(GemmCase("fc1_dx_nt", 64, 120, 256, 2, ("normal", 1.0), _kaiming(256)))
    cases.append(GemmCase("fc1_dw_tn", 256, 64, 120, 1, ("normal", 1.0), ("normal", 1.0)))
    return tuple(cases)


def _build() -> Dict[str, Workload]:
    lenet1 = ConvShape(8, 1, 28, 28, 5, 5, 1, 0, 6)
    lenet2 = ConvShape(64, 6, 12, 12, 5, 5, 1, 0, 16)
    alex1 = ConvShape(32, 3, 224, 224, 11, 11, 4, 2, 96)
    alex3 = ConvShape(64, 256, 13, 13, 3, 3, 1, 1, 384)
    alex4 = ConvShape(64, 384, 13, 13, 3, 3, 1, 1, 384)
    alex5 = ConvShape(64, 384, 13, 13, 3, 3, 1, 1, 256)
    fm3 = ConvShape(4, 256, 46, 80, 3, 3, 1, 1, 256)
    fm1 = ConvShape(4, 256, 46, 80, 1, 1, 1, 0, 128)
    fm3s2 = ConvShape(4, 256, 46, 80, 3, 3, 2, 1, 128)
    relu = ("relu_normal",)
    w = {
        "c1": Workload("c1", 1, "LeNet conv1, batch 8", ("f32",), (
            ConvLayer("conv1", lenet1, ("uniform", 0.0, 1.0), ("normal", 0.1)),)),
        "c2": Workload("c2", 2, "LeNet conv2 + FC GEMMs, batch 64", ("f32",), (
            ConvLayer("conv2", lenet2, ("normal", 1.0), _kaiming(lenet2.Kc)),),
            _fc_cases()),
        "c3": Workload("c3", 3, "AlexNet conv1 11x11 s4 p2, batch 32", ("f32",), (
            ConvLayer("conv1", alex1, ("uniform", 0.0, 1.0), _kaiming(alex1.Kc)),)),
        "c4": Workload("c4", 4, "AlexNet conv3-5 stack at 13x13, batch 64", ("f32", "bf16"), (
            ConvLayer("conv3", alex3, relu, _kaiming(alex3.Kc)),
            ConvLayer("conv4", alex4, relu, _kaiming(alex4.Kc)),
            ConvLayer("conv5", alex5, relu, _kaiming(alex5.Kc)),)),
        "c5": Workload("c5", 5, "Feature-map convs at 256x46x80, batch 4", ("f16",), (
            ConvLayer("conv3x3", fm3, ("normal", 1.0), ("normal", 1.0 / np.sqrt(fm3.Kc))),
            ConvLayer("conv1x1", fm1, ("normal", 1.0), ("normal", 1.0 / np.sqrt(fm1.Kc))),
            ConvLayer("conv3x3s2", fm3s2, ("normal", 1.0), ("normal", 1.0 / np.sqrt(fm3s2.Kc))),)),
    }
    return w


WORKLOADS: Dict[str, Workload] = _build()


# ----------------------------------------------------------------------------
# Seeded generation and dtype rounding
# ----------------------------------------------------------------------------

def draw(dist: tuple, shape, seed: tuple) -> np.ndarray:
    """Draw float64 values for ``dist`` with a generator seeded by ``seed``."""
    rng = np.random.default_rng(seed)
    kind = dist[0]
    if kind == "uniform":
        v = rng.uniform(dist[1], dist[2], size=shape)
    elif kind == "normal":
        v = rng.normal(0.0, dist[1], size=shape)
    elif kind == "relu_normal":
        v = np.maximum(rng.normal(0.0, 1.0, size=shape), 0.0)
    elif kind == "iota":
        v = np.arange(1, int(np.prod(shape)) + 1, dtype=np.float64).reshape(shape)
    elif kind == "small_int":
        v = rng.integers(-dist[1], dist[1] + 1, size=shape).astype(np.float64)
    elif kind == "dyadic":
        # integers in [lo, hi] scaled by 2^-frac: exact in float32, and so are
        # short sums and products of them
        v = rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float64) * 2.0 ** -dist[3]
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return v


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Operand:
    """One input tensor in a storage dtype.

    ``stored`` holds what goes to the device: float32 values, or uint16 bit
    patterns for float16/bfloat16.  ``exact`` is the same values widened
    exactly to float64, which is what the oracle consumes.
    """
    dtype: str
    stored: np.ndarray
    exact: np.ndarray


def quantize(v64: np.ndarray, dtype: str) -> Operand:
    v32 = v64.astype(np.float32)
    if dtype == "f32":
        return Operand("f32", v32, v32.astype(np.float64))
    if dtype == "f16":
        h = v32.astype(np.float16)
        return Operand("f16", h.view(np.uint16), h.astype(np.float64))
    if dtype == "bf16":
        bits = f32_to_bf16_bits(v32)
        return Operand("bf16", bits, bf16_bits_to_f64(bits))
    raise ValueError(dtype)


def conv_inputs(wl: Workload, layer_idx: int, dtype: str,
                batch: Optional[int] = None) -> Dict[str, Operand]:
    """x, W, g in ``dtype`` and bias in f32 for one conv layer of a workload.

    ``batch`` takes the leading images of the full-size draw, so a sample is
    a prefix of the same tensors the full run uses.
    """
    layer = wl.layers[layer_idx]
    s = layer.shape
    seed = lambda t: (wl.cfg_id, layer_idx, t)
    x = draw(layer.x_dist, s.x_shape(), seed(TID_X))
    w = draw(layer.w_dist, s.w_shape(), seed(TID_W))
    b = draw(layer.b_dist, (s.outC,), seed(TID_B))
    g = draw(layer.g_dist, s.y_shape(), seed(TID_G))
    if batch is not None:
        x, g = x[:batch], g[:batch]
    return {"x": quantize(x, dtype), "w": quantize(w, dtype),
            "bias": quantize(b, "f32"), "g": quantize(g, dtype)}


def gemm_inputs(wl: Workload, case_idx: int, dtype: str) -> Dict[str, Operand]:
    """A and B for a GEMM case, in the storage layout its flags name."""
    c = wl.gemms[case_idx]
    a = draw(c.a_dist, (c.M, c.K), (wl.cfg_id, 100 + case_idx, TID_A))
    b = draw(c.b_dist, (c.K, c.N), (wl.cfg_id, 100 + case_idx, TID_BM))
    a_st = a.T.copy() if c.flags & 1 else a
    b_st = b.T.copy() if c.flags & 2 else b
    return {"A": quantize(np.ascontiguousarray(a_st), dtype),
            "B": quantize(np.ascontiguousarray(b_st), dtype)}


def random_conv(shape: ConvShape, dtype: str, seed: int,
                x_dist=("normal", 1.0), w_dist=("normal", 1.0)) -> Dict[str, Operand]:
    """Inputs for an ad-hoc shape (edge-case tests)."""
    x = draw(x_dist, shape.x_shape(), (9000 + seed, 0, TID_X))
    w = draw(w_dist, shape.w_shape(), (9000 + seed, 0, TID_W))
    b = draw(("normal", 0.01), (shape.outC,), (9000 + seed, 0, TID_B))
    g = draw(("normal", 1.0), shape.y_shape(), (9000 + seed, 0, TID_G))
    return {"x": quantize(x, dtype), "w": quantize(w, dtype),
            "bias": quantize(b, "f32"), "g": quantize(g, dtype)}


# ----------------------------------------------------------------------------
# The rest of a training step: activations, labels, a LeNet-5 step
# ----------------------------------------------------------------------------

def f32_array(dist: tuple, shape, seed: tuple) -> np.ndarray:
    """``draw`` rounded to float32 (the storage of every training-step op)."""
    return draw(dist, shape, seed).astype(np.float32)


def labels(rows: int, classes: int, seed: tuple) -> np.ndarray:
    """Uniform class labels in [0, classes), int32."""
    return np.random.default_rng(seed).integers(0, classes, size=rows).astype(np.int32)


# LeNet-5 of the directcompute-nn page ("File Structure": 1->6->16 conv,
# 256->120->84->10 FC) on 1x28x28 inputs: conv 5x5 (no padding), ReLU, max
# pool 2x2 stride 2, twice, then three linear layers with ReLU between.
LENET_PARAMS = (("conv1_w", (6, 1, 5, 5)), ("conv1_b", (6,)),
                ("conv2_w", (16, 6, 5, 5)), ("conv2_b", (16,)),
                ("fc1_w", (120, 256)), ("fc1_b", (120,)),
                ("fc2_w", (84, 120)), ("fc2_b", (84,)),
                ("fc3_w", (10, 84)), ("fc3_b", (10,)))


def lenet_step_inputs(batch: int, seed: int) -> Dict[str, np.ndarray]:
    """Seeded float32 inputs of one LeNet-5 training step.

    The image and the convolution parameters are small dyadic rationals, so
    the convolutions, ReLUs and poolings are exact in float32 and every
    max-pool choice (ties included) is the same in any precision.  Linear
    layers are Kaiming-normal, biases small normal.  x is a binarised digit
    stand-in (values 0 or 1 on a 28x28 plane); labels are uniform in 0..9.
    """
    out: Dict[str, np.ndarray] = {}
    out["x"] = f32_array(("dyadic", 0, 1, 0), (batch, 1, 28, 28), (900 + seed, 0))
    out["labels"] = labels(batch, 10, (900 + seed, 1))
    dists = {"conv1_w": ("dyadic", -2, 2, 2), "conv1_b": ("dyadic", -1, 1, 2),
             "conv2_w": ("dyadic", -2, 2, 4), "conv2_b": ("dyadic", -1, 1, 4),
             "fc1_w": _kaiming(256), "fc2_w": _kaiming(120), "fc3_w": _kaiming(84)}
    for t, (name, shape) in enumerate(LENET_PARAMS):
        out[name] = f32_array(dists.get(name, ("normal", 0.01)), shape, (900 + seed, 2 + t))
    return out


# AlexNet as the directcompute-nn page trains it on PetImages ("File
# Structure": 5 conv layers, 3 FC layers; two classes), with the layer sizes
# of the AlexNet configs above: conv1 3->96 11x11 s4 p2 (224 -> 55), ReLU,
# max pool 3x3 s2 (-> 27); conv2 96->256 5x5 p2, ReLU, pool (-> 13); conv3
# 256->384, conv4 384->384, conv5 384->256 (3x3 p1), ReLU after each, pool
# after conv5 (-> 6); flatten to 9216; linear 9216->4096, ReLU, 4096->4096,
# ReLU, 4096->2.
ALEXNET_CLASSES = 2
ALEXNET_PARAMS = (("conv1_w", (96, 3, 11, 11)), ("conv1_b", (96,)),
                  ("conv2_w", (256, 96, 5, 5)), ("conv2_b", (256,)),
                  ("conv3_w", (384, 256, 3, 3)), ("conv3_b", (384,)),
                  ("conv4_w", (384, 384, 3, 3)), ("conv4_b", (384,)),
                  ("conv5_w", (256, 384, 3, 3)), ("conv5_b", (256,)),
                  ("fc1_w", (4096, 9216)), ("fc1_b", (4096,)),
                  ("fc2_w", (4096, 4096)), ("fc2_b", (4096,)),
                  ("fc3_w", (ALEXNET_CLASSES, 4096)), ("fc3_b", (ALEXNET_CLASSES,)))


def alexnet_step_inputs(batch: int, seed: int) -> Dict[str, np.ndarray]:
    """Seeded float32 inputs of one AlexNet training step.

    x is U[0, 1) on 3x224x224 (the AlexNet conv1 config's input); every
    weight is Kaiming-normal for its fan-in, biases N(0, 0.01); labels are
    uniform over the two classes.
    """
    out: Dict[str, np.ndarray] = {}
    out["x"] = f32_array(("uniform", 0.0, 1.0), (batch, 3, 224, 224), (950 + seed, 0))
    out["labels"] = labels(batch, ALEXNET_CLASSES, (950 + seed, 1))
    for t, (name, shape) in enumerate(ALEXNET_PARAMS):
        fan_in = int(np.prod(shape[1:]))
        dist = _kaiming(fan_in) if name.endswith("_w") else ("normal", 0.01)
        out[name] = f32_array(dist, shape, (950 + seed, 2 + t))
    return out

