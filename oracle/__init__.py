"""Python binding of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may import this package.  The HIP library and its binding never do.

Every function takes and returns float64 numpy arrays in the layouts the
pages' convolution uses: x NCHW, W OIHW, y/g NCHW, col (C*kH*kW) x (B*OH*OW)
row-major; GEMM operands packed as the two transpose-flag index formulas
("Transpose via Flags", directcompute-nn page) describe.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into oracle/liboracle.so."""
    if not force and os.path.exists(LIB_PATH) and \
            os.path.getmtime(LIB_PATH) >= os.path.getmtime(SRC_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", "-o", tmp, SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run oracle.build() or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_longlong
        conv_args = [L] * 9
        lib.oracle_conv_forward.argtypes = [P, P, P, P] + conv_args
        lib.oracle_conv_backward_filter.argtypes = [P, P, P] + conv_args
        lib.oracle_conv_backward_data.argtypes = [P, P, P] + conv_args
        lib.oracle_conv_backward_bias.argtypes = [P, P, L, L, L]
        lib.oracle_gemm.argtypes = [P, P, P, L, L, L, ctypes.c_int]
        lib.oracle_im2col_spec.argtypes = [P, P] + [L] * 8
        lib.oracle_col2im_spec.argtypes = [P, P] + [L] * 8
        lib.oracle_out_dims.argtypes = [L] * 6 + [ctypes.POINTER(L)] * 2
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        I32 = ctypes.POINTER(ctypes.c_int32)
        D = ctypes.c_double
        lib.oracle_relu.argtypes = [P, P, L]
        lib.oracle_relu_grad.argtypes = [P, P, P, L]
        lib.oracle_maxpool_forward.argtypes = [P, P, I32] + [L] * 6
        lib.oracle_maxpool_backward.argtypes = [P, I32, P] + [L] * 6
        lib.oracle_add_bias_rows.argtypes = [P, P, P, L, L]
        lib.oracle_bias_grad_rows.argtypes = [P, P, L, L]
        lib.oracle_softmax.argtypes = [P, P, L, L]
        lib.oracle_softmax_ce_grad.argtypes = [P, I32, P, L, L]
        lib.oracle_ce_loss.argtypes = [P, I32, ctypes.POINTER(D), L, L]
        lib.oracle_sgd.argtypes = [P, P, L, D, D]
        lib.oracle_grad_accum.argtypes = [P, P, L]
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def out_dims(H: int, W: int, kH: int, kW: int, s: int, p: int) -> Tuple[int, int]:
    oh, ow = ctypes.c_longlong(), ctypes.c_longlong()
    rc = _load().oracle_out_dims(H, W, kH, kW, s, p, ctypes.byref(oh), ctypes.byref(ow))
    if rc != 0:
        raise ValueError("invalid convolution geometry")
    return int(oh.value), int(ow.value)


def _geom(x_shape, w_shape, stride, padding):
    B, C, H, W = x_shape
    O, C2, kH, kW = w_shape
    if C != C2:
        raise ValueError("channel mismatch between x and W")
    OH, OW = out_dims(H, W, kH, kW, stride, padding)
    if OH < 1 or OW < 1:
        raise ValueError("kernel larger than the padded input")
    return B, C, H, W, O, kH, kW, OH, OW


def conv_forward(x, w, bias=None, stride=1, padding=0) -> np.ndarray:
    """y = conv(x; W) + bias, direct summation over the kernel window."""
    x, w = _f64(x), _f64(w)
    B, C, H, W, O, kH, kW, OH, OW = _geom(x.shape, w.shape, stride, padding)
    b = None if bias is None else _f64(bias)
    y = np.empty((B, O, OH, OW), dtype=np.float64)
    rc = _load().oracle_conv_forward(_ptr(x), _ptr(w), _ptr(b), _ptr(y),
                                     B, C, H, W, O, kH, kW, stride, padding)
    if rc != 0:
        raise ValueError("oracle_conv_forward rejected the shape")
    return y


def conv_backward_filter(x, g, w_shape, stride=1, padding=0) -> np.ndarray:
    x, g = _f64(x), _f64(g)
    B, C, H, W, O, kH, kW, OH, OW = _geom(x.shape, w_shape, stride, padding)
    if g.shape != (B, O, OH, OW):
        raise ValueError("g shape mismatch")
    dw = np.empty((O, C, kH, kW), dtype=np.float64)
    rc = _load().oracle_conv_backward_filter(_ptr(x), _ptr(g), _ptr(dw),
                                             B, C, H, W, O, kH, kW, stride, padding)
    if rc != 0:
        raise ValueError("oracle_conv_backward_filter rejected the shape")
    return dw


def conv_backward_bias(g) -> np.ndarray:
    g = _f64(g)
    B, O = g.shape[0], g.shape[1]
    P = int(np.prod(g.shape[2:]))
    db = np.empty((O,), dtype=np.float64)
    rc = _load().oracle_conv_backward_bias(_ptr(g), _ptr(db), B, O, P)
    if rc != 0:
        raise ValueError("oracle_conv_backward_bias rejected the shape")
    return db


def conv_backward_data(g, w, x_shape, stride=1, padding=0) -> np.ndarray:
    g, w = _f64(g), _f64(w)
    B, C, H, W, O, kH, kW, OH, OW = _geom(x_shape, w.shape, stride, padding)
    if g.shape != (B, O, OH, OW):
        raise ValueError("g shape mismatch")
    dx = np.empty((B, C, H, W), dtype=np.float64)
    rc = _load().oracle_conv_backward_data(_ptr(g), _ptr(w), _ptr(dx),
                                           B, C, H, W, O, kH, kW, stride, padding)
    if rc != 0:
        raise ValueError("oracle_conv_backward_data rejected the shape")
    return dx


def gemm(A, Bm, M: int, K: int, N: int, flags: int) -> np.ndarray:
    """C[M,N] = op(A) op(B) from packed storage, per the flag index formulas."""
    A, Bm = _f64(A).reshape(-1), _f64(Bm).reshape(-1)
    if A.size != M * K or Bm.size != K * N:
        raise ValueError("operand size mismatch")
    C = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(_ptr(A), _ptr(Bm), _ptr(C), M, K, N, int(flags))
    if rc != 0:
        raise ValueError("oracle_gemm rejected the arguments")
    return C


def im2col_spec(x, kH: int, kW: int, stride: int, padding: int) -> np.ndarray:
    x = _f64(x)
    B, C, H, W = x.shape
    OH, OW = out_dims(H, W, kH, kW, stride, padding)
    col = np.empty((C * kH * kW, B * OH * OW), dtype=np.float64)
    rc = _load().oracle_im2col_spec(_ptr(x), _ptr(col), B, C, H, W, kH, kW,
                                    stride, padding)
    if rc != 0:
        raise ValueError("oracle_im2col_spec rejected the shape")
    return col


def col2im_spec(col, x_shape, kH: int, kW: int, stride: int, padding: int) -> np.ndarray:
    col = _f64(col)
    B, C, H, W = x_shape
    OH, OW = out_dims(H, W, kH, kW, stride, padding)
    if col.shape != (C * kH * kW, B * OH * OW):
        raise ValueError("col shape mismatch")
    dx = np.empty((B, C, H, W), dtype=np.float64)
    rc = _load().oracle_col2im_spec(_ptr(col), _ptr(dx), B, C, H, W, kH, kW,
                                    stride, padding)
    if rc != 0:
        raise ValueError("oracle_col2im_spec rejected the shape")
    return dx



# ---------------------------------------------------------------------------
# the rest of a training step ("HLSL Shader Reference": activation / loss,
# pooling and utility shaders of the directcompute-nn page)
# ---------------------------------------------------------------------------

def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle_{what} rejected its arguments")


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def relu(x) -> np.ndarray:
    x = _f64(x)
    y = np.empty_like(x)
    _check(_load().oracle_relu(_ptr(x), _ptr(y), x.size), "relu")
    return y


def relu_grad(x, dy) -> np.ndarray:
    x, dy = _f64(x), _f64(dy)
    dx = np.empty_like(x)
    _check(_load().oracle_relu_grad(_ptr(x), _ptr(dy), _ptr(dx), x.size), "relu_grad")
    return dx


def pool_dims(H: int, W: int, k: int, s: int) -> Tuple[int, int]:
    return (H - k) // s + 1, (W - k) // s + 1


def maxpool_forward(x, k: int, s: int) -> Tuple[np.ndarray, np.ndarray]:
    """(y, idx): idx is the offset h*W + w of the maximum inside its plane."""
    x = _f64(x)
    B, C, H, W = x.shape
    OH, OW = pool_dims(H, W, k, s)
    y = np.empty((B, C, OH, OW))
    idx = np.empty((B, C, OH, OW), dtype=np.int32)
    _check(_load().oracle_maxpool_forward(_ptr(x), _ptr(y), _iptr(idx), B, C, H, W, k, s),
           "maxpool_forward")
    return y, idx


def maxpool_backward(dy, idx, x_shape, k: int, s: int) -> np.ndarray:
    dy, idx = _f64(dy), _i32(idx)
    B, C, H, W = x_shape
    dx = np.empty((B, C, H, W))
    _check(_load().oracle_maxpool_backward(_ptr(dy), _iptr(idx), _ptr(dx), B, C, H, W, k, s),
           "maxpool_backward")
    return dx


def add_bias_rows(x, bias) -> np.ndarray:
    x, bias = _f64(x), _f64(bias)
    rows, cols = x.shape
    y = np.empty_like(x)
    _check(_load().oracle_add_bias_rows(_ptr(x), _ptr(bias), _ptr(y), rows, cols), "add_bias_rows")
    return y


def bias_grad_rows(dy) -> np.ndarray:
    dy = _f64(dy)
    rows, cols = dy.shape
    db = np.empty(cols)
    _check(_load().oracle_bias_grad_rows(_ptr(dy), _ptr(db), rows, cols), "bias_grad_rows")
    return db


def softmax(z) -> np.ndarray:
    z = _f64(z)
    rows, classes = z.shape
    p = np.empty_like(z)
    _check(_load().oracle_softmax(_ptr(z), _ptr(p), rows, classes), "softmax")
    return p


def softmax_ce_grad(z, labels) -> np.ndarray:
    z, labels = _f64(z), _i32(labels)
    rows, classes = z.shape
    dz = np.empty_like(z)
    _check(_load().oracle_softmax_ce_grad(_ptr(z), _iptr(labels), _ptr(dz), rows, classes),
           "softmax_ce_grad")
    return dz


def ce_loss(z, labels) -> float:
    z, labels = _f64(z), _i32(labels)
    rows, classes = z.shape
    out = ctypes.c_double()
    _check(_load().oracle_ce_loss(_ptr(z), _iptr(labels), ctypes.byref(out), rows, classes), "ce_loss")
    return out.value


def sgd(param, grad, lr: float, clip: float) -> np.ndarray:
    """Returns the updated parameter (the input array is not modified)."""
    p = _f64(param).copy()
    g = _f64(grad)
    _check(_load().oracle_sgd(_ptr(p), _ptr(g), p.size, float(lr), float(clip)), "sgd")
    return p


def grad_accum(acc, grad) -> np.ndarray:
    a = _f64(acc).copy()
    g = _f64(grad)
    _check(_load().oracle_grad_accum(_ptr(a), _ptr(g), a.size), "grad_accum")
    return a


# ---------------------------------------------------------------------------
# One LeNet-5 training step composed from the functions above
# ---------------------------------------------------------------------------

def lenet_step(inp: dict, lr: float, clip: float) -> dict:
    """Forward, backward and SGD update of LeNet-5 on one batch, in float64.

    The network is the directcompute-nn page's LeNet ("File Structure":
    1->6->16 conv, 256->120->84->10 FC) on 1x28x28 images: conv 5x5 without
    padding, ReLU, max pool 2x2 stride 2, twice; flatten (NCHW order) to 256;
    linear 256->120, ReLU, 120->84, ReLU, 84->10; softmax-cross-entropy.
    Each layer follows the page's autograd ("Autograd"; "Convolution: The
    im2col Approach" for the conv gradients, "Transpose via Flags" for the
    linear ones): a linear layer y = x W^T + b (W stored out x in) is the
    matmul with flags 2; its data gradient dy W is flags 0 and its weight
    gradient dy^T x is flags 1.  The loss gradient is softmax - one_hot (no
    1/batch factor); the first convolution's data gradient is not needed.
    Every parameter then takes param -= lr * clamp(grad, -clip, clip).

    ``inp`` holds x, labels and the parameters named in workloads.LENET_PARAMS.
    Returns the loss, every activation, every gradient (key "d" + name) and
    every updated parameter (key "new_" + name).
    """
    f = {k: _f64(v) if k != "labels" else np.asarray(v) for k, v in inp.items()}
    B = f["x"].shape[0]
    r = {}
    # forward
    r["a1"] = relu(conv_forward(f["x"], f["conv1_w"], f["conv1_b"], 1, 0))          # B,6,24,24
    r["p1"], r["idx1"] = maxpool_forward(r["a1"], 2, 2)                              # B,6,12,12
    r["a2"] = relu(conv_forward(r["p1"], f["conv2_w"], f["conv2_b"], 1, 0))         # B,16,8,8
    r["p2"], r["idx2"] = maxpool_forward(r["a2"], 2, 2)                              # B,16,4,4
    flat = r["p2"].reshape(B, 256)
    r["pre1"] = add_bias_rows(gemm(flat, f["fc1_w"], B, 256, 120, 2), f["fc1_b"])
    r["h1"] = relu(r["pre1"])
    r["pre2"] = add_bias_rows(gemm(r["h1"], f["fc2_w"], B, 120, 84, 2), f["fc2_b"])
    r["h2"] = relu(r["pre2"])
    r["z"] = add_bias_rows(gemm(r["h2"], f["fc3_w"], B, 84, 10, 2), f["fc3_b"])
    r["loss"] = ce_loss(r["z"], f["labels"])
    # backward
    dz = softmax_ce_grad(r["z"], f["labels"])
    r["dz"] = dz
    r["dfc3_w"] = gemm(dz, r["h2"], 10, B, 84, 1)
    r["dfc3_b"] = bias_grad_rows(dz)
    dh2 = relu_grad(r["pre2"], gemm(dz, f["fc3_w"], B, 10, 84, 0))
    r["dfc2_w"] = gemm(dh2, r["h1"], 84, B, 120, 1)
    r["dfc2_b"] = bias_grad_rows(dh2)
    dh1 = relu_grad(r["pre1"], gemm(dh2, f["fc2_w"], B, 84, 120, 0))
    r["dfc1_w"] = gemm(dh1, flat, 120, B, 256, 1)
    r["dfc1_b"] = bias_grad_rows(dh1)
    dflat = gemm(dh1, f["fc1_w"], B, 120, 256, 0)
    da2 = maxpool_backward(dflat.reshape(r["p2"].shape), r["idx2"], r["a2"].shape, 2, 2)
    g2 = relu_grad(r["a2"], da2)
    r["dconv2_w"] = conv_backward_filter(r["p1"], g2, f["conv2_w"].shape, 1, 0)
    r["dconv2_b"] = conv_backward_bias(g2)
    dp1 = conv_backward_data(g2, f["conv2_w"], r["p1"].shape, 1, 0)
    da1 = maxpool_backward(dp1, r["idx1"], r["a1"].shape, 2, 2)
    g1 = relu_grad(r["a1"], da1)
    r["dconv1_w"] = conv_backward_filter(f["x"], g1, f["conv1_w"].shape, 1, 0)
    r["dconv1_b"] = conv_backward_bias(g1)
    # update
    for name in ("conv1_w", "conv1_b", "conv2_w", "conv2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b",
                 "fc3_w", "fc3_b"):
        r["new_" + name] = sgd(f[name], r["d" + name], lr, clip)
    return r


def alexnet_step(inp: dict, lr: float, clip: float) -> dict:
    """Forward, backward and SGD update of AlexNet on one batch, in float64.

    The directcompute-nn page trains AlexNet on two-class PetImages ("File
    Structure": 5 conv layers, 3 FC layers), with the same autograd rules as
    lenet_step.  Layers (sizes of the AlexNet configs): conv1 11x11 stride 4
    pad 2, ReLU, max pool 3x3 stride 2; conv2 5x5 pad 2, ReLU, pool; conv3,
    conv4, conv5 3x3 pad 1 with ReLU after each and a pool after conv5;
    flatten (NCHW order) to 9216; linear 9216->4096, ReLU, 4096->4096, ReLU,
    4096->classes; softmax-cross-entropy (gradient softmax - one_hot, no
    1/batch factor); param -= lr * clamp(grad, -clip, clip).

    ``inp`` holds x, labels and the parameters named in
    workloads.ALEXNET_PARAMS.  Returns the loss, the activations ("a1".."a5"
    ReLU outputs, "p1", "p2", "p5" pooled, "h1", "h2", "z"), every gradient
    ("d" + name) and every updated parameter ("new_" + name).
    """
    f = {k: _f64(v) if k != "labels" else np.asarray(v) for k, v in inp.items()}
    B = f["x"].shape[0]
    r = {}
    # forward: (input, stride, padding, pool after)
    convs = (("conv1", "x", 4, 2, True), ("conv2", "p1", 1, 2, True), ("conv3", "p2", 1, 1, False),
             ("conv4", "a3", 1, 1, False), ("conv5", "a4", 1, 1, True))
    src = {"x": f["x"]}
    for i, (name, inp_key, s, p, pool) in enumerate(convs, start=1):
        a = relu(conv_forward(src[inp_key], f[name + "_w"], f[name + "_b"], s, p))
        r["a%d" % i] = src["a%d" % i] = a
        if pool:
            r["p%d" % i], r["idx%d" % i] = maxpool_forward(a, 3, 2)
            src["p%d" % i] = r["p%d" % i]
    flat = r["p5"].reshape(B, -1)
    n_in, n_h, n_out = flat.shape[1], f["fc1_w"].shape[0], f["fc3_w"].shape[0]
    r["pre1"] = add_bias_rows(gemm(flat, f["fc1_w"], B, n_in, n_h, 2), f["fc1_b"])
    r["h1"] = relu(r["pre1"])
    r["pre2"] = add_bias_rows(gemm(r["h1"], f["fc2_w"], B, n_h, n_h, 2), f["fc2_b"])
    r["h2"] = relu(r["pre2"])
    r["z"] = add_bias_rows(gemm(r["h2"], f["fc3_w"], B, n_h, n_out, 2), f["fc3_b"])
    r["loss"] = ce_loss(r["z"], f["labels"])
    # backward
    dz = softmax_ce_grad(r["z"], f["labels"])
    r["dz"] = dz
    r["dfc3_w"] = gemm(dz, r["h2"], n_out, B, n_h, 1)
    r["dfc3_b"] = bias_grad_rows(dz)
    dh2 = relu_grad(r["pre2"], gemm(dz, f["fc3_w"], B, n_out, n_h, 0))
    r["dfc2_w"] = gemm(dh2, r["h1"], n_h, B, n_h, 1)
    r["dfc2_b"] = bias_grad_rows(dh2)
    dh1 = relu_grad(r["pre1"], gemm(dh2, f["fc2_w"], B, n_h, n_h, 0))
    r["dfc1_w"] = gemm(dh1, flat, n_h, B, n_in, 1)
    r["dfc1_b"] = bias_grad_rows(dh1)
    dflat = gemm(dh1, f["fc1_w"], B, n_h, n_in, 0)
    # the gradient reaching each conv layer's ReLU output, from the top
    d = maxpool_backward(dflat.reshape(r["p5"].shape), r["idx5"], r["a5"].shape, 3, 2)
    for i in (5, 4, 3, 2, 1):
        name, inp_key, s, p, _ = convs[i - 1]
        g = relu_grad(r["a%d" % i], d)
        x_in = src[inp_key]
        r["d%s_w" % name] = conv_backward_filter(x_in, g, f[name + "_w"].shape, s, p)
        r["d%s_b" % name] = conv_backward_bias(g)
        if i == 1:
            break
        d = conv_backward_data(g, f[name + "_w"], x_in.shape, s, p)
        if inp_key.startswith("p"):  # through the pool that produced this input
            k = int(inp_key[1:])
            d = maxpool_backward(d, r["idx%d" % k], r["a%d" % k].shape, 3, 2)
    # update
    for name in [n for n in inp if n not in ("x", "labels")]:
        r["new_" + name] = sgd(f[name], r["d" + name], lr, clip)
    return r

