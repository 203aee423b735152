"""Python binding of libd4r_conv: convolution lowered to GEMM on MI355X.

Argument marshalling only.  Every function named ``d4r_*`` calls the C entry
point of the same name (declared in ``include/d4r_conv.h``); tensors are
passed as device pointers and the stream is torch's current stream.  All
arithmetic runs in the library's HIP kernels; nothing here computes.  The
library must be built (``python gemm_scratch_nn_amd/build.py``); importing
this package without it raises ImportError.

``ConvPlan`` wraps one handle and allocates outputs and the workspace with
``torch.empty`` (device memory plumbing, no compute).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libd4r_conv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "d4r_conv.h")

D4R_F32, D4R_F16, D4R_BF16 = 0, 1, 2
DTYPE_NAMES = {D4R_F32: "f32", D4R_F16: "f16", D4R_BF16: "bf16"}
STATUS = {0: "D4R_OK", 1: "D4R_ERR_INVALID_ARG", 2: "D4R_ERR_UNSUPPORTED",
          3: "D4R_ERR_WORKSPACE", 4: "D4R_ERR_LAUNCH", 5: "D4R_ERR_INTERNAL"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python gemm_scratch_nn_amd/build.py` (hipcc, gfx950)")

# torch must be loaded first: it ships its own libamdhip64.so.7, and the
# library's libamdhip64.so.7 dependency must resolve to that same runtime
# (device buffers and streams come from torch).  Loading this library first
# would map a second HIP runtime into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def hip_runtimes(maps_text: str) -> set:
    """Paths of the libamdhip64 files mapped, from /proc/<pid>/maps text."""
    return {ln.split()[-1] for ln in maps_text.splitlines() if "libamdhip64" in ln}


def check_single_hip_runtime(maps_text: str) -> None:
    """ImportError when the maps show two HIP runtimes (every launch would fail)."""
    found = hip_runtimes(maps_text)
    if len(found) > 1:
        raise ImportError("two HIP runtimes are mapped into this process "
                          f"({sorted(found)}); import torch before anything "
                          "that loads /opt/rocm's libamdhip64")


try:
    with open("/proc/self/maps") as _maps:
        _maps_text = _maps.read()
except OSError:
    _maps_text = ""
check_single_hip_runtime(_maps_text)

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_ll = ctypes.c_longlong
_f = ctypes.c_float
_st = ctypes.c_int


def _sig(name, args, res=_st):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_c = {
    "d4r_conv_create": _sig("d4r_conv_create", [ctypes.POINTER(_vp)] + [_i] * 9 + [_i]),
    "d4r_conv_destroy": _sig("d4r_conv_destroy", [_vp]),
    "d4r_conv_output_dims": _sig("d4r_conv_output_dims", [_vp, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "d4r_conv_workspace_size": _sig("d4r_conv_workspace_size", [_vp, ctypes.POINTER(_sz)]),
    "d4r_conv_describe": _sig("d4r_conv_describe", [_vp, ctypes.c_char_p, _sz, ctypes.POINTER(_sz)]),
    "d4r_conv_forward": _sig("d4r_conv_forward", [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_conv_forward_implicit": _sig("d4r_conv_forward_implicit",
                                      [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_conv_forward_ex": _sig("d4r_conv_forward_ex", [_vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "d4r_conv_backward_data": _sig("d4r_conv_backward_data", [_vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_conv_backward_data_implicit": _sig("d4r_conv_backward_data_implicit",
                                            [_vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_conv_packed_filter_size": _sig("d4r_conv_packed_filter_size", [_vp, ctypes.POINTER(_sz)]),
    "d4r_conv_pack_filter": _sig("d4r_conv_pack_filter", [_vp, _vp, _vp, _vp]),
    "d4r_conv_backward_data_packed": _sig("d4r_conv_backward_data_packed",
                                          [_vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_conv_backward_filter": _sig("d4r_conv_backward_filter",
                                     [_vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "d4r_conv_backward": _sig("d4r_conv_backward", [_vp] * 7 + [_i, _vp, _sz, _vp]),
    "d4r_conv_im2col": _sig("d4r_conv_im2col", [_vp, _vp, _vp, _vp]),
    "d4r_conv_col2im": _sig("d4r_conv_col2im", [_vp, _vp, _vp, _vp]),
    "d4r_conv_bias_grad": _sig("d4r_conv_bias_grad", [_vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_gemm_workspace_size": _sig("d4r_gemm_workspace_size", [_i, _i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "d4r_gemm": _sig("d4r_gemm", [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "d4r_gemm_noalloc": _sig("d4r_gemm_noalloc", [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "d4r_gemm_noalloc_scratch_bytes": _sig("d4r_gemm_noalloc_scratch_bytes", [], _sz),
    "d4r_gemm_bias_act": _sig("d4r_gemm_bias_act", [_i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "d4r_relu_forward": _sig("d4r_relu_forward", [_vp, _vp, _ll, _vp]),
    "d4r_relu_backward": _sig("d4r_relu_backward", [_vp, _vp, _vp, _ll, _vp]),
    "d4r_maxpool_forward": _sig("d4r_maxpool_forward", [_vp, _vp, _vp] + [_i] * 6 + [_vp]),
    "d4r_maxpool_backward": _sig("d4r_maxpool_backward", [_vp, _vp, _vp] + [_i] * 6 + [_vp]),
    "d4r_add_bias_rows": _sig("d4r_add_bias_rows", [_vp, _vp, _vp, _i, _i, _vp]),
    "d4r_bias_grad_rows": _sig("d4r_bias_grad_rows", [_vp, _vp, _i, _i, _vp]),
    "d4r_softmax": _sig("d4r_softmax", [_vp, _vp, _i, _i, _vp]),
    "d4r_softmax_ce_grad": _sig("d4r_softmax_ce_grad", [_vp, _vp, _vp, _vp, _i, _i, _vp]),
    "d4r_sgd_update": _sig("d4r_sgd_update", [_vp, _vp, _ll, _f, _f, _vp]),
    "d4r_grad_accum": _sig("d4r_grad_accum", [_vp, _vp, _ll, _vp]),
    "d4r_stream_copy": _sig("d4r_stream_copy", [_vp, _vp, _sz, _vp]),
    "d4r_stream_fill": _sig("d4r_stream_fill", [_vp, ctypes.c_uint, _sz, _vp]),
    "d4r_mfma_ceiling": _sig("d4r_mfma_ceiling", [ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp]),
    "d4r_profile_enable": _sig("d4r_profile_enable", [_i]),
    "d4r_profile_reset": _sig("d4r_profile_reset", []),
    "d4r_status_string": _sig("d4r_status_string", [_i], ctypes.c_char_p),
    "d4r_last_error": _sig("d4r_last_error", [], ctypes.c_char_p),
}


class d4r_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int), ("ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_c["d4r_profile_read"] = _sig("d4r_profile_read",
                              [ctypes.POINTER(d4r_kernel_stat), _i, ctypes.POINTER(_i)])


class D4RError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.fn = fn
        self.status = status
        self.msg = msg


def _check(fn: str, st: int) -> None:
    if st != 0:
        msg = _c["d4r_last_error"]().decode(errors="replace")
        raise D4RError(fn, st, msg)


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor, or an int / None passed through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        raise TypeError("pass ws_bytes explicitly with a raw workspace pointer")
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def declared_functions() -> list:
    """Names of the functions include/d4r_conv.h declares."""
    with open(HEADER_PATH) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(d4r_[a-z0-9_]+)\s*\(", src)))


def exported(name: str) -> bool:
    return hasattr(_lib, name)


# ---------------------------------------------------------------------------
# One Python function per C entry point (same names, same argument order).
# ---------------------------------------------------------------------------

def d4r_status_string(status: int) -> str:
    return _c["d4r_status_string"](status).decode()


def d4r_last_error() -> str:
    return _c["d4r_last_error"]().decode(errors="replace")


def d4r_conv_create(batch, inC, inH, inW, kH, kW, stride, padding, outC, dtype) -> int:
    h = _vp()
    _check("d4r_conv_create", _c["d4r_conv_create"](ctypes.byref(h), batch, inC, inH, inW,
                                                    kH, kW, stride, padding, outC, dtype))
    return h.value


def d4r_conv_destroy(h) -> None:
    _check("d4r_conv_destroy", _c["d4r_conv_destroy"](h))


def d4r_conv_output_dims(h) -> Tuple[int, int]:
    oh, ow = _i(), _i()
    _check("d4r_conv_output_dims", _c["d4r_conv_output_dims"](h, ctypes.byref(oh), ctypes.byref(ow)))
    return oh.value, ow.value


def d4r_conv_workspace_size(h) -> int:
    n = _sz()
    _check("d4r_conv_workspace_size", _c["d4r_conv_workspace_size"](h, ctypes.byref(n)))
    return n.value


def d4r_conv_describe(h) -> dict:
    """The handle's launch plan as a dict of the key=value pairs the C call returns."""
    need = _sz()
    _check("d4r_conv_describe", _c["d4r_conv_describe"](h, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check("d4r_conv_describe", _c["d4r_conv_describe"](h, buf, need.value, ctypes.byref(need)))
    return dict(kv.split("=", 1) for kv in buf.value.decode().split())


def d4r_conv_forward(h, x, w, bias, y, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_forward", _c["d4r_conv_forward"](h, _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                                                      _ptr(ws), nb, _stream(stream)))


def d4r_conv_forward_implicit(h, x, w, bias, y, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_forward_implicit",
           _c["d4r_conv_forward_implicit"](h, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(ws), nb,
                                           _stream(stream)))


D4R_FWD_RELU, D4R_FWD_IMPLICIT = 1, 2


def d4r_conv_forward_ex(h, x, w, bias, y, flags, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_forward_ex",
           _c["d4r_conv_forward_ex"](h, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), int(flags), _ptr(ws), nb,
                                     _stream(stream)))


def d4r_conv_backward_data(h, w, dy, dx, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_backward_data", _c["d4r_conv_backward_data"](h, _ptr(w), _ptr(dy), _ptr(dx),
                                                                  _ptr(ws), nb, _stream(stream)))


def d4r_conv_backward_data_implicit(h, w, dy, dx, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_backward_data_implicit",
           _c["d4r_conv_backward_data_implicit"](h, _ptr(w), _ptr(dy), _ptr(dx), _ptr(ws), nb,
                                                 _stream(stream)))


def d4r_conv_packed_filter_size(h) -> int:
    n = _sz()
    _check("d4r_conv_packed_filter_size", _c["d4r_conv_packed_filter_size"](h, ctypes.byref(n)))
    return n.value


def d4r_conv_pack_filter(h, w, wp, stream=None) -> None:
    _check("d4r_conv_pack_filter", _c["d4r_conv_pack_filter"](h, _ptr(w), _ptr(wp), _stream(stream)))


def d4r_conv_backward_data_packed(h, wp, dy, dx, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_backward_data_packed",
           _c["d4r_conv_backward_data_packed"](h, _ptr(wp), _ptr(dy), _ptr(dx), _ptr(ws), nb, _stream(stream)))


def d4r_conv_backward_filter(h, x, dy, dw, db, reuse_col, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_backward_filter",
           _c["d4r_conv_backward_filter"](h, _ptr(x), _ptr(dy), _ptr(dw), _ptr(db), int(reuse_col),
                                          _ptr(ws), nb, _stream(stream)))


def d4r_conv_backward(h, x, w, dy, dx, dw, db, reuse_col, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_backward",
           _c["d4r_conv_backward"](h, _ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db), int(reuse_col),
                                   _ptr(ws), nb, _stream(stream)))


def d4r_conv_im2col(h, x, col, stream=None) -> None:
    _check("d4r_conv_im2col", _c["d4r_conv_im2col"](h, _ptr(x), _ptr(col), _stream(stream)))


def d4r_conv_col2im(h, dcol, dx, stream=None) -> None:
    _check("d4r_conv_col2im", _c["d4r_conv_col2im"](h, _ptr(dcol), _ptr(dx), _stream(stream)))


def d4r_conv_bias_grad(h, dy, db, ws, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_conv_bias_grad", _c["d4r_conv_bias_grad"](h, _ptr(dy), _ptr(db), _ptr(ws), nb,
                                                          _stream(stream)))


def d4r_gemm_workspace_size(M, K, N, flags, dtype) -> int:
    n = _sz()
    _check("d4r_gemm_workspace_size", _c["d4r_gemm_workspace_size"](M, K, N, flags, dtype, ctypes.byref(n)))
    return n.value


def d4r_gemm(M, K, N, flags, dtype, A, B, C, ws=None, ws_bytes=None, stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_gemm", _c["d4r_gemm"](M, K, N, flags, dtype, _ptr(A), _ptr(B), _ptr(C), _ptr(ws), nb,
                                      _stream(stream)))


def d4r_gemm_noalloc(M, K, N, flags, dtype, A, B, C, stream=None) -> None:
    _check("d4r_gemm_noalloc", _c["d4r_gemm_noalloc"](M, K, N, flags, dtype, _ptr(A), _ptr(B), _ptr(C),
                                                      _stream(stream)))


def d4r_gemm_noalloc_scratch_bytes() -> int:
    return int(_c["d4r_gemm_noalloc_scratch_bytes"]())


def d4r_gemm_bias_act(M, K, N, flags, dtype, A, B, bias, relu, C, ws=None, ws_bytes=None,
                      stream=None) -> None:
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check("d4r_gemm_bias_act",
           _c["d4r_gemm_bias_act"](M, K, N, flags, dtype, _ptr(A), _ptr(B), _ptr(bias), int(relu), _ptr(C),
                                   _ptr(ws), nb, _stream(stream)))


def d4r_relu_forward(x, y, n, stream=None) -> None:
    _check("d4r_relu_forward", _c["d4r_relu_forward"](_ptr(x), _ptr(y), n, _stream(stream)))


def d4r_relu_backward(x, dy, dx, n, stream=None) -> None:
    _check("d4r_relu_backward", _c["d4r_relu_backward"](_ptr(x), _ptr(dy), _ptr(dx), n, _stream(stream)))


def d4r_maxpool_forward(x, y, idx, batch, channels, H, W, k, stride, stream=None) -> None:
    _check("d4r_maxpool_forward", _c["d4r_maxpool_forward"](_ptr(x), _ptr(y), _ptr(idx), batch, channels, H, W,
                                                            k, stride, _stream(stream)))


def d4r_maxpool_backward(dy, idx, dx, batch, channels, H, W, k, stride, stream=None) -> None:
    _check("d4r_maxpool_backward", _c["d4r_maxpool_backward"](_ptr(dy), _ptr(idx), _ptr(dx), batch, channels,
                                                              H, W, k, stride, _stream(stream)))


def d4r_add_bias_rows(x, bias, y, rows, cols, stream=None) -> None:
    _check("d4r_add_bias_rows", _c["d4r_add_bias_rows"](_ptr(x), _ptr(bias), _ptr(y), rows, cols,
                                                        _stream(stream)))


def d4r_bias_grad_rows(dy, db, rows, cols, stream=None) -> None:
    _check("d4r_bias_grad_rows", _c["d4r_bias_grad_rows"](_ptr(dy), _ptr(db), rows, cols, _stream(stream)))


def d4r_softmax(z, p, rows, classes, stream=None) -> None:
    _check("d4r_softmax", _c["d4r_softmax"](_ptr(z), _ptr(p), rows, classes, _stream(stream)))


def d4r_softmax_ce_grad(z, labels, dz, loss, rows, classes, stream=None) -> None:
    _check("d4r_softmax_ce_grad", _c["d4r_softmax_ce_grad"](_ptr(z), _ptr(labels), _ptr(dz), _ptr(loss), rows,
                                                            classes, _stream(stream)))


def d4r_sgd_update(param, grad, n, lr, clip, stream=None) -> None:
    _check("d4r_sgd_update", _c["d4r_sgd_update"](_ptr(param), _ptr(grad), n, lr, clip, _stream(stream)))


def d4r_grad_accum(acc, grad, n, stream=None) -> None:
    _check("d4r_grad_accum", _c["d4r_grad_accum"](_ptr(acc), _ptr(grad), n, _stream(stream)))


def d4r_stream_copy(dst, src, nbytes, stream=None) -> None:
    _check("d4r_stream_copy", _c["d4r_stream_copy"](_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def d4r_stream_fill(dst, value, nbytes, stream=None) -> None:
    _check("d4r_stream_fill", _c["d4r_stream_fill"](_ptr(dst), int(value) & 0xFFFFFFFF, nbytes,
                                                    _stream(stream)))


def d4r_mfma_ceiling(dtype: int, src, out, blocks: int, iters: int, stream=None) -> None:
    _check("d4r_mfma_ceiling", _c["d4r_mfma_ceiling"](dtype, _ptr(src), _ptr(out), blocks, iters, _stream(stream)))


def d4r_profile_enable(on: bool) -> None:
    _check("d4r_profile_enable", _c["d4r_profile_enable"](1 if on else 0))


def d4r_profile_reset() -> None:
    _check("d4r_profile_reset", _c["d4r_profile_reset"]())


def d4r_profile_read() -> list:
    """Per kernel class: dict(name, launches, ms, flops, bytes).  Synchronises."""
    n = _i()
    _check("d4r_profile_read", _c["d4r_profile_read"](None, 0, ctypes.byref(n)))
    buf = (d4r_kernel_stat * max(1, n.value))()
    _check("d4r_profile_read", _c["d4r_profile_read"](buf, n.value, ctypes.byref(n)))
    return [{"name": buf[i].name.decode(), "launches": buf[i].launches, "ms": buf[i].ms,
             "flops": buf[i].flops, "bytes": buf[i].bytes} for i in range(n.value)]


# ---------------------------------------------------------------------------
# Convenience wrapper: one handle, outputs and workspace allocated by torch.
# ---------------------------------------------------------------------------

def torch_dtype_code(t) -> int:
    import torch
    m = {torch.float32: D4R_F32, torch.float16: D4R_F16, torch.bfloat16: D4R_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _require(t, name, dtype_code=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype_code is not None and torch_dtype_code(t) != dtype_code:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {DTYPE_NAMES[dtype_code]}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class ConvPlan:
    """A convolution handle plus torch-allocated workspace."""

    def __init__(self, batch, inC, inH, inW, kH, kW, stride, padding, outC, dtype: int,
                 device="cuda"):
        import torch
        self.shape = (batch, inC, inH, inW, kH, kW, stride, padding, outC)
        self.dtype = dtype
        self.h = d4r_conv_create(batch, inC, inH, inW, kH, kW, stride, padding, outC, dtype)
        self.outH, self.outW = d4r_conv_output_dims(self.h)
        self.ws_bytes = d4r_conv_workspace_size(self.h)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.device = device

    def describe(self) -> dict:
        """The launch plan of this handle (d4r_conv_describe)."""
        return d4r_conv_describe(self.h)

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            self.h = None
            try:
                d4r_conv_destroy(h)
            except Exception:  # interpreter shutdown: the binding may be gone
                pass

    @property
    def x_shape(self):
        b, c, hh, ww = self.shape[:4]
        return (b, c, hh, ww)

    @property
    def w_shape(self):
        return (self.shape[8], self.shape[1], self.shape[4], self.shape[5])

    @property
    def y_shape(self):
        return (self.shape[0], self.shape[8], self.outH, self.outW)

    @property
    def Kc(self):
        return self.shape[1] * self.shape[4] * self.shape[5]

    @property
    def N(self):
        return self.shape[0] * self.outH * self.outW

    def forward(self, x, w, bias=None, y=None):
        import torch
        _require(x, "x", self.dtype, self.x_shape)
        _require(w, "w", self.dtype, self.w_shape)
        if bias is not None:
            _require(bias, "bias", D4R_F32, (self.shape[8],))
        if y is None:
            y = torch.empty(self.y_shape, dtype=torch.float32, device=x.device)
        d4r_conv_forward(self.h, x, w, bias, y, self.ws, self.ws_bytes)
        return y

    def forward_implicit(self, x, w, bias=None, y=None):
        import torch
        _require(x, "x", self.dtype, self.x_shape)
        _require(w, "w", self.dtype, self.w_shape)
        if bias is not None:
            _require(bias, "bias", D4R_F32, (self.shape[8],))
        if y is None:
            y = torch.empty(self.y_shape, dtype=torch.float32, device=x.device)
        d4r_conv_forward_implicit(self.h, x, w, bias, y, self.ws, self.ws_bytes)
        return y

    def forward_relu(self, x, w, bias=None, y=None, implicit=False):
        """y = relu(conv(x; w) + bias) in one GEMM epilogue (d4r_conv_forward_ex)."""
        import torch
        _require(x, "x", self.dtype, self.x_shape)
        _require(w, "w", self.dtype, self.w_shape)
        if bias is not None:
            _require(bias, "bias", D4R_F32, (self.shape[8],))
        if y is None:
            y = torch.empty(self.y_shape, dtype=torch.float32, device=x.device)
        d4r_conv_forward_ex(self.h, x, w, bias, y, D4R_FWD_RELU | (D4R_FWD_IMPLICIT if implicit else 0),
                            self.ws, self.ws_bytes)
        return y

    def backward_data(self, w, dy, dx=None):
        import torch
        _require(w, "w", self.dtype, self.w_shape)
        _require(dy, "dy", self.dtype, self.y_shape)
        if dx is None:
            dx = torch.empty(self.x_shape, dtype=torch.float32, device=dy.device)
        d4r_conv_backward_data(self.h, w, dy, dx, self.ws, self.ws_bytes)
        return dx

    def backward_data_implicit(self, w, dy, dx=None):
        import torch
        _require(w, "w", self.dtype, self.w_shape)
        _require(dy, "dy", self.dtype, self.y_shape)
        if dx is None:
            dx = torch.empty(self.x_shape, dtype=torch.float32, device=dy.device)
        d4r_conv_backward_data_implicit(self.h, w, dy, dx, self.ws, self.ws_bytes)
        return dx

    def pack_filter(self, w, wp=None):
        """The data gradient's packed filter (Kc x O) for backward_data_packed."""
        import torch
        _require(w, "w", self.dtype, self.w_shape)
        if wp is None:
            wp = torch.empty((self.Kc, self.shape[8]), dtype=w.dtype, device=w.device)
        d4r_conv_pack_filter(self.h, w, wp)
        return wp

    def backward_data_packed(self, wp, dy, dx=None):
        import torch
        _require(wp, "wp", self.dtype, (self.Kc, self.shape[8]))
        _require(dy, "dy", self.dtype, self.y_shape)
        if dx is None:
            dx = torch.empty(self.x_shape, dtype=torch.float32, device=dy.device)
        d4r_conv_backward_data_packed(self.h, wp, dy, dx, self.ws, self.ws_bytes)
        return dx

    def backward_filter(self, x, dy, reuse_col=False, want_bias=True, dw=None, db=None):
        import torch
        if not reuse_col:
            _require(x, "x", self.dtype, self.x_shape)
        _require(dy, "dy", self.dtype, self.y_shape)
        if dw is None:
            dw = torch.empty(self.w_shape, dtype=torch.float32, device=dy.device)
        if want_bias and db is None:
            db = torch.empty((self.shape[8],), dtype=torch.float32, device=dy.device)
        d4r_conv_backward_filter(self.h, None if reuse_col else x, dy, dw, db if want_bias else None,
                                 1 if reuse_col else 0, self.ws, self.ws_bytes)
        return dw, (db if want_bias else None)

    def backward(self, x, w, dy, reuse_col=False, want_bias=True, dx=None, dw=None, db=None):
        """dx, dw, db of one layer through d4r_conv_backward."""
        import torch
        if not reuse_col:
            _require(x, "x", self.dtype, self.x_shape)
        _require(w, "w", self.dtype, self.w_shape)
        _require(dy, "dy", self.dtype, self.y_shape)
        if dx is None:
            dx = torch.empty(self.x_shape, dtype=torch.float32, device=dy.device)
        if dw is None:
            dw = torch.empty(self.w_shape, dtype=torch.float32, device=dy.device)
        if want_bias and db is None:
            db = torch.empty((self.shape[8],), dtype=torch.float32, device=dy.device)
        d4r_conv_backward(self.h, None if reuse_col else x, w, dy, dx, dw, db if want_bias else None,
                          1 if reuse_col else 0, self.ws, self.ws_bytes)
        return dx, dw, (db if want_bias else None)

    def col_view(self):
        """The col matrix the last forward / im2col left at the start of ws."""
        import torch
        es = 4 if self.dtype == D4R_F32 else 2
        n = self.Kc * self.N
        raw = self.ws[: n * es]
        tdt = {D4R_F32: torch.float32, D4R_F16: torch.float16, D4R_BF16: torch.bfloat16}[self.dtype]
        return raw.view(tdt).view(self.Kc, self.N)


def gemm(A, B, M, K, N, flags, C=None):
    """C = op(A) op(B) through d4r_gemm; allocates C and any workspace."""
    import torch
    dt = torch_dtype_code(A)
    _require(A, "A", dt)
    _require(B, "B", dt)
    if A.numel() != M * K or B.numel() != K * N:
        raise ValueError("operand sizes do not match M, K, N")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    wsb = d4r_gemm_workspace_size(M, K, N, flags, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=A.device) if wsb else None
    d4r_gemm(M, K, N, flags, dt, A, B, C, ws, wsb)
    return C
