"""GPU-side adjoint identities of the convolution, independent of the oracle.

The forward y = conv(x; W) is linear in x and in W, and the gradients are
its adjoints: <y, g> = <x, dx> = <W, dW>, and sum(db) = sum(g) (the page's
"Convolution: The im2col Approach" forward and backward; the identities
follow from the definitions alone).  Every workload layer runs through the
library: forward without bias, the default data gradient (implicit where the
planner takes it, else dcol + col2im) and the filter gradient, also through
the combined backward.  The inner products are taken in float64 on the host
from the GPU's outputs and the exact (dtype-rounded) inputs.  Inputs are
exact in their dtype and the GEMMs accumulate in f32, so the identities hold
to f32 rounding; the bound (1e-4 of the summed absolute terms) is loose for
that, while a wrong index, tap, flip or transpose breaks them by order one.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import workloads as wl
from gpu_util import DT_CODE, dev, host

pytestmark = pytest.mark.gpu

# (workload, dtype, batch): every layer of each workload at that batch
CASES = [("c1", "f32", 8), ("c2", "f32", 64), ("c3", "f32", 2), ("c4", "f32", 4), ("c4", "bf16", 4),
         ("c5", "f16", 1), ("c4", "f32", 64)]


def _dot(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b), float(np.abs(a) @ np.abs(b))


@pytest.mark.parametrize("key,dt,batch", CASES, ids=[f"{k}-{d}-b{b}" for k, d, b in CASES])
def test_adjoint_identities_on_gpu(key, dt, batch):
    w_ = wl.WORKLOADS[key]
    for li, layer in enumerate(w_.layers):
        sh = layer.shape.with_batch(batch)
        ops = wl.conv_inputs(w_, li, dt, batch=batch)
        x, w, g = dev(ops["x"]), dev(ops["w"]), dev(ops["g"])
        pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding, sh.outC,
                          DT_CODE[dt])
        y = pl.forward(x, w)
        dx = pl.backward_data_implicit(w, g)
        dw, db = pl.backward_filter(x, g, reuse_col=False)
        dx2, dw2, db2 = pl.backward(x, w, g, reuse_col=False)
        torch.cuda.synchronize()
        X, W, G = ops["x"].exact, ops["w"].exact, ops["g"].exact
        yg, yg_abs = _dot(host(y), G)
        for tag, (DX, DW, DB) in {"separate": (dx, dw, db), "combined": (dx2, dw2, db2)}.items():
            xdx, xdx_abs = _dot(X, host(DX))
            wdw, wdw_abs = _dot(W, host(DW))
            scale = max(yg_abs, xdx_abs, wdw_abs)
            print(f"adjoint {key} {dt} b{batch} layer {li} {tag}: <y,g>={yg:.6e} <x,dx>={xdx:.6e} "
                  f"<W,dW>={wdw:.6e} rel {abs(yg - xdx) / scale:.1e} {abs(yg - wdw) / scale:.1e}", flush=True)
            assert abs(yg - xdx) <= 1e-4 * scale, (li, tag, "x", yg, xdx)
            assert abs(yg - wdw) <= 1e-4 * scale, (li, tag, "W", yg, wdw)
            sg = float(np.asarray(G, dtype=np.float64).sum())
            sg_abs = float(np.abs(np.asarray(G, dtype=np.float64)).sum())
            assert abs(float(host(DB).astype(np.float64).sum()) - sg) <= 1e-5 * sg_abs, (li, tag, "b")
