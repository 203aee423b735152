"""HIP-graph capture and replay of a whole conv forward + backward.

Every library call only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a step can be captured
with stream capture and replayed.  Each replay runs after eager work that
changes the inputs in place, and is checked against an eager run on the
same inputs.
"""
import numpy as np
import pytest
import torch

import gemm_scratch_nn_amd as d4r
import workloads as wl
from gpu_util import DT_CODE, dev

pytestmark = pytest.mark.gpu


def _setup(key, li, dt, batch):
    w = wl.WORKLOADS[key]
    sh = w.layers[li].shape.with_batch(batch)
    ops = wl.conv_inputs(w, li, dt, batch=batch)
    pl = d4r.ConvPlan(sh.batch, sh.inC, sh.inH, sh.inW, sh.kH, sh.kW, sh.stride, sh.padding, sh.outC,
                      DT_CODE[dt])
    t = {k: dev(ops[k]) for k in ("x", "w", "g", "bias")}
    t["y"] = torch.empty(sh.y_shape(), dtype=torch.float32, device="cuda")
    t["dx"] = torch.empty(sh.x_shape(), dtype=torch.float32, device="cuda")
    t["dw"] = torch.empty(sh.w_shape(), dtype=torch.float32, device="cuda")
    t["db"] = torch.empty((sh.outC,), dtype=torch.float32, device="cuda")
    return pl, t


def _step(pl, t, stream):
    d4r.d4r_conv_forward(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, stream)
    d4r.d4r_conv_backward_data(pl.h, t["w"], t["g"], t["dx"], pl.ws, pl.ws_bytes, stream)
    d4r.d4r_conv_backward_filter(pl.h, None, t["g"], t["dw"], t["db"], 1, pl.ws, pl.ws_bytes, stream)


@pytest.mark.parametrize("key,li,dt,batch", [("c1", 0, "f32", 8), ("c2", 0, "f32", 64),
                                             ("c4", 1, "bf16", 4), ("c5", 2, "f16", 1)])
def test_graph_replay_matches_eager(key, li, dt, batch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pl, t = _setup(key, li, dt, batch)
    _step(pl, t, torch.cuda.current_stream().cuda_stream)   # warm up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(pl, t, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(4):
        # eager work between replays: new input values, in place
        t["x"].mul_(-0.5 if r % 2 else 1.25)
        t["g"].add_(0.125)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: t[k].clone() for k in ("y", "dx", "dw", "db")}
        _step(pl, t, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], t[k]), (r, k)


@pytest.mark.parametrize("key,li,dt,batch", [("c4", 1, "f32", 4), ("c4", 2, "bf16", 4), ("c5", 1, "f16", 1)])
def test_gradients_on_two_streams_match_one_stream(key, li, dt, batch):
    # the data gradient (its own workspace) on a second stream, overlapping
    # the filter gradient that reuses the forward's col: results equal the
    # one-stream sequence bit for bit (the library only enqueues; nothing is
    # shared between the two besides the read-only w and dy)
    pl, t = _setup(key, li, dt, batch)
    main = torch.cuda.current_stream()
    _step(pl, t, main.cuda_stream)
    torch.cuda.synchronize()
    ref = {k: t[k].clone() for k in ("y", "dx", "dw", "db")}
    for k in ("y", "dx", "dw", "db"):
        t[k].fill_(float("nan"))
    ws2 = torch.empty(pl.ws_bytes, dtype=torch.uint8, device="cuda")
    aux = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        d4r.d4r_conv_forward(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, main.cuda_stream)
        aux.wait_stream(main)
        d4r.d4r_conv_backward_data(pl.h, t["w"], t["g"], t["dx"], ws2, pl.ws_bytes, aux.cuda_stream)
        d4r.d4r_conv_backward_filter(pl.h, None, t["g"], t["dw"], t["db"], 1, pl.ws, pl.ws_bytes,
                                     main.cuda_stream)
        main.wait_stream(aux)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(ref[k], t[k]), k


@pytest.mark.parametrize("key,li,dt,batch", [("c4", 1, "f32", 4), ("c4", 2, "bf16", 4)])
def test_graph_replay_combined_backward(key, li, dt, batch):
    # the combined backward (one dy preparation launch for both gradients)
    # captured once and replayed after in-place input changes
    pl, t = _setup(key, li, dt, batch)

    def step():
        st = torch.cuda.current_stream().cuda_stream  # the capture stream inside the graph block
        d4r.d4r_conv_forward(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, st)
        d4r.d4r_conv_backward(pl.h, None, t["w"], t["g"], t["dx"], t["dw"], t["db"], 1, pl.ws, pl.ws_bytes, st)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        t["x"].mul_(-0.5 if r % 2 else 1.25)
        t["g"].add_(0.125)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: t[k].clone() for k in ("y", "dx", "dw", "db")}
        step()
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], t[k]), (r, k)


@pytest.mark.parametrize("key,li,dt,batch,implicit", [("c5", 1, "f16", 1, True), ("c4", 0, "bf16", 4, True),
                                                      ("c5", 2, "f16", 1, False), ("c3", 0, "f32", 2, False)])
def test_graph_replay_bench_step_forms(key, li, dt, batch, implicit):
    # the step forms the bench times: the 1x1 in-place forward and the NHWC
    # forward with the combined backward redoing im2col (implicit), and the
    # explicit forward whose col the combined backward reuses (the phased
    # data gradient on the stride-2 layer, the one-pass explicit backward on
    # AlexNet conv1)
    pl, t = _setup(key, li, dt, batch)

    def step():
        st = torch.cuda.current_stream().cuda_stream
        if implicit:
            d4r.d4r_conv_forward_implicit(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, st)
            d4r.d4r_conv_backward(pl.h, t["x"], t["w"], t["g"], t["dx"], t["dw"], t["db"], 0, pl.ws, pl.ws_bytes,
                                  st)
        else:
            d4r.d4r_conv_forward(pl.h, t["x"], t["w"], t["bias"], t["y"], pl.ws, pl.ws_bytes, st)
            d4r.d4r_conv_backward(pl.h, None, t["w"], t["g"], t["dx"], t["dw"], t["db"], 1, pl.ws, pl.ws_bytes,
                                  st)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        t["x"].mul_(-0.5 if r % 2 else 1.25)
        t["g"].add_(0.125)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: t[k].clone() for k in ("y", "dx", "dw", "db")}
        step()
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], t[k]), (r, k)
